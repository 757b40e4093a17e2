"""The allocation-free attention entry point, csa2_sparse_attn_decode_static,
against csa2_sparse_attn_decode with a caller workspace: two calls in a row,
the second with a smaller input (the static scratch still holds the first
call's partials), bit-identical results (the same kernels and split count),
and the oracle's tolerance on sampled sequences."""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_kv_amd import csa2
from decode_kv_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, lens, k, Hq, window=128):
    rng = np.random.default_rng(seed)
    B = len(lens)
    row_off = [int(x) for x in np.cumsum([0] + lens[:-1])]
    codes_t, scales_t = W.raw_fp4_rows(seed, max(1, sum(lens)), 512, 118, 130)
    sel = np.full((B, k), -1, dtype=np.int32)
    sel_len = []
    for b, L in enumerate(lens):
        E = max(0, L - window)
        m = min(k, E)
        if m:
            sel[b, :m] = np.sort(rng.choice(E, m, replace=False))
        sel_len.append(m)
    q = (rng.standard_normal((B, Hq, 512)).astype(np.float32).view(np.uint32) >> 16) \
        .astype(np.uint16)
    return dict(codes=codes_t.numpy(), scales=scales_t.numpy(), row_off=row_off, lens=lens,
                sel=sel, sel_len=sel_len, q=q, k=k, window=window)


def _run(inp, static: bool):
    B, Hq, D = inp["q"].shape
    k, window = inp["k"], inp["window"]
    args = (torch.from_numpy(inp["q"].view(np.int16)).to(DEV).view(torch.bfloat16),
            torch.from_numpy(inp["codes"]).to(DEV), torch.from_numpy(inp["scales"]).to(DEV),
            torch.tensor(inp["row_off"], dtype=torch.int64, device=DEV),
            torch.tensor(inp["lens"], dtype=torch.int32, device=DEV), max(inp["lens"]),
            torch.from_numpy(inp["sel"]).to(DEV),
            torch.tensor(inp["sel_len"], dtype=torch.int32, device=DEV), k, window,
            1 / math.sqrt(D))
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    if static:
        csa2.sparse_attn_decode_static(*args, out, lse)
    else:
        ws = csa2.workspace(csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, B, 0, 0, 0, 0, k, Hq, D,
                                                 window))
        csa2.sparse_attn_decode(*args, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_oracle(inp, out, lse, seqs):
    for b in seqs:
        L = inp["lens"][b]
        S = oracle.attention_positions(L, inp["sel"][b, :inp["sel_len"][b]], inp["window"])
        rows = inp["row_off"][b] + S
        ro, rl = oracle.attention(inp["q"][b], inp["codes"][rows], inp["scales"][rows],
                                  1 / math.sqrt(512))
        m = np.abs(ro).max()
        assert np.abs(out[b].astype(np.float64) - ro).max() <= 1e-3 * m, b
        assert (np.abs(lse[b] - rl) <= 1e-3 + 1e-6 * np.abs(rl)).all(), b


def test_static_scratch_matches_workspace_variant():
    rng = np.random.default_rng(5)
    big = _inputs(51, [int(x) for x in rng.integers(700, 5000, size=32)], 512, 64)
    small = _inputs(52, [3000, 129, 2500], 512, 64)
    one = _inputs(53, [4096], 512, 64)
    need = csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, 32, 0, 0, 0, 0, 512, 64, 512, 128)
    assert 16 << 20 < need <= csa2.ATTN_STATIC_SCRATCH_BYTES      # most of the scratch
    for name, inp, seqs in [("32 sequences", big, [0, 17, 31]), ("3 sequences", small, [0, 1, 2]),
                            ("1 sequence", one, [0])]:
        print(name, flush=True)
        out_ws, lse_ws = _run(inp, static=False)
        out_st, lse_st = _run(inp, static=True)
        assert np.array_equal(out_ws, out_st, equal_nan=True), name
        assert np.array_equal(lse_ws, lse_st, equal_nan=True), name
        _check_oracle(inp, out_st, lse_st, seqs)


def test_static_scratch_rejects_oversized_inputs():
    """64 sequences x 64 heads need 42 MB of partials: rejected before launch,
    and the outputs stay untouched."""
    B, Hq = 64, 64
    q = torch.zeros((B, Hq, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((8, 256), dtype=torch.uint8, device=DEV)
    sc = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    ro = torch.zeros(B, dtype=torch.int64, device=DEV)
    ln = torch.full((B,), 8, dtype=torch.int32, device=DEV)
    sel = torch.full((B, 512), -1, dtype=torch.int32, device=DEV)
    sl = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = torch.full((B, Hq, 512), 7.0, device=DEV)
    with pytest.raises(csa2.Csa2Error) as ei:
        csa2.sparse_attn_decode_static(q, kv, sc, ro, ln, 8, sel, sl, 512, 128, 0.04, out, None)
    assert ei.value.code == csa2.CSA2_ERR_UNSUPPORTED and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
