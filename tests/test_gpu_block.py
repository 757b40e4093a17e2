"""GPU parity of the verify-block entry points (T drafted tokens per sequence,
per-token or shared selection) against the oracle's block functions, on the
same seeded inputs.  Same bar as the one-token path: pools, selections and
scores bit-exact, attention within 1e-3 * max|out|."""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_kv_amd import csa2, pipeline
from decode_kv_amd import workloads as W
from test_gpu_parity import DEV, _say, check_attention, u16

pytestmark = pytest.mark.gpu


def _keys(rng, n, kind):
    if kind == "ties":                     # few distinct scores: ties at every boundary
        return rng.integers(-1, 2, size=(n, 64)).astype(np.int8)
    return rng.integers(-127, 128, size=(n, 64)).astype(np.int8)


def _block_case(seed, lens, T, H=64, kind="uniform"):
    rng = np.random.default_rng(seed)
    B = len(lens)
    row_off = [0] + list(np.cumsum(lens)[:-1])
    keys = _keys(rng, max(1, sum(lens)), kind)
    hi = 2 if kind == "ties" else 128
    q = rng.integers(-hi + 1, hi, size=(B, T, H, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=(B, T, H)).astype(np.int8)
    return keys, [int(x) for x in row_off], q, w


def _t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_full_block(keys, row_off, lens, q, w, window, P, k, shared):
    B, T = q.shape[:2]
    nl = B if shared else B * T
    pos = torch.full((nl, P), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    scr = torch.full((nl, P), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    plen = torch.full((nl,), -9, dtype=torch.int32, device=DEV)
    sel = torch.full((nl, max(k, 1)), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    slen = torch.full((nl,), -9, dtype=torch.int32, device=DEV)
    max_len, total_len = max(lens), keys.shape[0]
    ws = csa2.workspace(csa2.block_workspace_bytes(csa2.OP_INDEX_FULL, B, T, shared, max_len,
                                                   total_len, q.shape[2], P, k))
    ro = torch.tensor(row_off, dtype=torch.int64, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    csa2.index_full_block(_t(q), _t(w), _t(keys), ro, ln, max_len, total_len, window, P, shared,
                          pos, scr, plen, ws, k=k, sel_pos=sel if k else None,
                          sel_len=slen if k else None)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (pos, scr, plen, sel, slen)]


def check_full_block(keys, row_off, lens, q, w, window, P, k, shared, what=""):
    pos, scr, plen, sel, slen = run_full_block(keys, row_off, lens, q, w, window, P, k, shared)
    T = q.shape[1]
    for b, L in enumerate(lens):
        ref = oracle.index_full_block(keys, row_off[b], L, T, q[b], w[b], window, P, shared)
        refs = [ref] if shared else ref
        for t, (rp, rs) in enumerate(refs):
            v = b if shared else b * T + t
            n = len(rp)
            tag = (what, b, t, L)
            assert plen[v] == n, tag
            assert np.array_equal(pos[v, :n], rp), tag
            assert np.array_equal(scr[v, :n], rs), tag
            assert (pos[v, n:] == -1).all() and (scr[v, n:] == -1).all(), tag
            if k:
                rsel, _ = oracle.select_topk(rs, rp, k)
                m = len(rsel)
                assert slen[v] == m and np.array_equal(sel[v, :m], rsel), tag
                assert (sel[v, m:k] == -1).all(), tag


@pytest.mark.parametrize("shared", [False, True])
def test_index_full_block_ragged(shared):
    """Lengths around tile edges (1,024 positions) and the window, one
    sequence shorter than a tile, one whose first tokens see nothing, one
    where no token ranks a position (no tiles: its lists' states come from
    workgroup 0)."""
    lens = [70000, 1024 + 128 + 2, 3 * 1024 + 128 + 4, 140, 133, 130, 100]
    keys, row_off, q, w = _block_case(1, lens, 5)
    check_full_block(keys, row_off, lens, q, w, 128, 2048, 100, shared, "ragged")


@pytest.mark.parametrize("shared", [False, True])
def test_index_full_block_ties(shared):
    lens = [20000, 5000]
    keys, row_off, q, w = _block_case(2, lens, 5, kind="ties")
    check_full_block(keys, row_off, lens, q, w, 128, 1500, 64, shared, "ties")


@pytest.mark.parametrize("shared", [False, True])
def test_index_full_block_sizes(shared):
    """T = 1 (the one-token call's results), T = 8 (the largest block), few
    heads (one, two and three blocks of 16), a pool larger than the context,
    k = 0."""
    lens = [9000, 300]
    keys, row_off, q, w = _block_case(3, lens, 1)
    check_full_block(keys, row_off, lens, q, w, 128, 1024, 64, shared, "T=1")
    keys, row_off, q, w = _block_case(4, lens, 8, H=4)
    check_full_block(keys, row_off, lens, q, w, 128, 16384, 512, shared, "T=8 H=4")
    keys, row_off, q, w = _block_case(5, lens, 3, H=20)
    check_full_block(keys, row_off, lens, q, w, 16, 777, 0, shared, "k=0")
    keys, row_off, q, w = _block_case(9, lens, 5, H=40)
    check_full_block(keys, row_off, lens, q, w, 128, 3000, 100, shared, "H=40")


def test_index_full_block_single_long_sequence():
    """One 1M-position sequence (the single-sequence code path) in both modes."""
    lens = [1 << 20]
    keys, row_off, q, w = _block_case(6, lens, 5)
    for shared in (False, True):
        check_full_block(keys, row_off, lens, q, w, 128, 16384, 512, shared, "1M")


@pytest.mark.parametrize("shared", [False, True])
def test_index_score_block(shared):
    lens = [5000, 1300, 131]
    keys, row_off, q, w = _block_case(7, lens, 5)
    B, T = q.shape[:2]
    max_len = max(lens)
    nl = B if shared else B * T
    score = torch.full((nl, max_len), -77, dtype=torch.int32, device=DEV)
    ws = csa2.workspace(csa2.block_workspace_bytes(csa2.OP_INDEX_FULL, B, T, shared, max_len,
                                                   keys.shape[0], 64, 1, 0))
    csa2.index_score_block(_t(q), _t(w), _t(keys), torch.tensor(row_off, device=DEV),
                           torch.tensor(lens, dtype=torch.int32, device=DEV), max_len,
                           keys.shape[0], 128, shared, score, ws)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    for b, L in enumerate(lens):
        Ls = oracle.block_lengths(L, T)
        if shared:
            E = oracle.eligible_count(Ls[0], 128)
            ref = np.max([oracle.index_scores(keys, row_off[b] + np.arange(E), q[b, t], w[b, t])
                          for t in range(T)], axis=0) if E else np.zeros(0, np.int64)
            assert np.array_equal(got[b, :E], ref) and (got[b, E:] == -77).all(), b
        else:
            for t in range(T):
                E = oracle.eligible_count(Ls[t], 128)
                ref = oracle.index_scores(keys, row_off[b] + np.arange(E), q[b, t], w[b, t])
                assert np.array_equal(got[b * T + t, :E], ref), (b, t)
                assert (got[b * T + t, E:] == -77).all(), (b, t)


@pytest.mark.parametrize("shared,T,H", [(False, 5, 64), (True, 2, 64), (True, 5, 64), (True, 9, 64),
                                        (True, 5, 20), (False, 3, 40)])
def test_index_reindex_block(shared, T, H):
    """A shared list's tokens are spread over the workgroup's four waves:
    T = 2 leaves two waves idle, T = 9 gives one wave three tokens; 20 and
    40 heads take the two- and three-block instances."""
    rng = np.random.default_rng(8 + T + H)
    lens = [200000, 6000]
    keys, row_off, q, w = _block_case(8, lens, T, H=H)
    B, P = 2, 16384
    nl = B if shared else B * T
    cand = np.full((nl, P), -1, dtype=np.int32)
    clen = []
    for v in range(nl):
        b = v if shared else v // T
        n = [16384, 4000, 1, 0, 9000][v % 5] if lens[b] > 100000 else 3000 - 7 * (v % 5)
        clen.append(n)
        if n:
            cand[v, :n] = np.sort(rng.choice(lens[b] - 128, n, replace=False))
    score = torch.full((nl, P), 0x7777, dtype=torch.int32, device=DEV)
    csa2.index_reindex_block(_t(q), _t(w), _t(keys), torch.tensor(row_off, device=DEV),
                             _t(cand), torch.tensor(clen, dtype=torch.int32, device=DEV), shared,
                             score)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    for v in range(nl):
        b = v if shared else v // T
        n = clen[v]
        if shared:
            ref = oracle.index_reindex_block(keys, row_off[b], cand[v, :n], q[b], w[b], True)
        else:
            t = v % T
            ref = oracle.index_reindex(keys, row_off[b], cand[v, :n], q[b, t], w[b, t])
        assert np.array_equal(got[v, :n], ref), v
        assert (got[v, n:] == -1).all(), v


@pytest.mark.parametrize("shared", [False, True])
def test_attention_block(shared):
    """Each token's own window and its (own or shared) selection; sequences
    shorter than the window and the block."""
    rng = np.random.default_rng(9)
    lens, T, k, Hq, window = [4096, 70000, 300, 129, 6], 5, 512, 64, 128
    B = len(lens)
    row_off = list(np.cumsum([0] + lens[:-1]))
    codes_t, scales_t = W.raw_fp4_rows(9, sum(lens), 512, 118, 130)
    codes, scales = codes_t.numpy(), scales_t.numpy()
    nl = B if shared else B * T
    sel = np.full((nl, k), -1, dtype=np.int32)
    slen = []
    for v in range(nl):
        b = v if shared else v // T
        t = 0 if shared else v % T
        E = oracle.eligible_count(oracle.block_lengths(lens[b], T)[t] if lens[b] >= T else 0,
                                  window)
        m = min(k, E)
        if m:
            sel[v, :m] = np.sort(rng.choice(E, m, replace=False))
        slen.append(m)
    qf = rng.standard_normal((B, T, Hq, 512)).astype(np.float32)
    qb = (qf.view(np.uint32) >> 16).astype(np.uint16)
    qt = torch.from_numpy(qb.view(np.int16)).to(DEV).view(torch.bfloat16)
    ws = csa2.workspace(csa2.block_workspace_bytes(csa2.OP_SPARSE_ATTN, B, T, shared, 0, 0, 0,
                                                   0, k, Hq, 512, window))
    out = torch.full((B, T, Hq, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    csa2.sparse_attn_decode_block(qt, _t(codes), _t(scales), torch.tensor(row_off, device=DEV),
                                  torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens),
                                  _t(sel), torch.tensor(slen, dtype=torch.int32, device=DEV), k,
                                  window, shared, 1 / math.sqrt(512), out, lse, ws)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b, L in enumerate(lens):
        for t in range(T):
            Lt = L - (T - 1 - t)
            v = b if shared else b * T + t
            if Lt <= 0:
                assert (out[b, t] == 0).all() and np.isneginf(lse[b, t]).all(), (b, t)
                continue
            S = oracle.attention_positions(Lt, sel[v, :slen[v]], window)
            rows = row_off[b] + S
            ro, rl = oracle.attention(qb[b, t], codes[rows], scales[rows], 1 / math.sqrt(512))
            check_attention(out[b, t], lse[b, t], ro, rl, "b %d t %d L %d" % (b, t, L))


# ---------------------------------------------------------------------------
# whole verify steps through the pipeline
# ---------------------------------------------------------------------------

def check_engine_block(eng, cpu_case, step, seqs, keys_np):
    wl = eng.wl
    T, sh = wl.block, wl.block_shared
    lens = cpu_case.lengths_at(step)
    FR = [l for l, c in enumerate(wl.pattern) if c in "FR"]
    for b in seqs:
        off = int(cpu_case.row_off[b])
        kb = keys_np[off:off + cpu_case.caps[b]]
        idx_q = {l: np.stack([cpu_case.index_q(step, l, b, t).numpy() for t in range(T)])
                 for l in FR}
        idx_w = {l: np.stack([cpu_case.index_w(step, l, b, t).numpy() for t in range(T)])
                 for l in FR}
        attn_q = [np.stack([u16(cpu_case.attn_q(step, l, b, t)) for t in range(T)])
                  for l in range(wl.n_layers)]
        res = oracle.decode_block(wl.pattern, kb, 0, lens[b], T, wl.window, wl.P, wl.k, idx_q,
                                  idx_w, attn_q, lambda l, S: u16(cpu_case.kv_bf16(l, b, S)),
                                  wl.sm_scale, sh)
        lists = [b] if sh else [b * T + t for t in range(T)]
        pools = [res[0]["pool_pos"]] if sh else res[0]["pool_pos"]
        pscores = [res[0]["pool_score"]] if sh else res[0]["pool_score"]
        for i, v in enumerate(lists):
            n = int(eng.pool_len[v])
            pool = eng.pool_pos[v].cpu().numpy()
            assert n == len(pools[i]) and np.array_equal(pool[:n], pools[i]), (step, b, i)
            assert np.array_equal(eng.pool_score[v].cpu().numpy()[:n], pscores[i]), (step, b, i)
            assert (pool[n:] == -1).all()
        for l, r in enumerate(res):
            src = eng.selection_layer(l)
            sels = [r["sel"]] if sh else r["sel"]
            for i, v in enumerate(lists):
                sl = int(eng.sel_len[src, v])
                assert sl == len(sels[i]), (step, b, l, i)
                assert np.array_equal(eng.sel_pos[src, v].cpu().numpy()[:sl], sels[i]), \
                    (step, b, l, i)
                if r["kind"] == "R":
                    rs = eng.rscore[l, v].cpu().numpy()
                    ref = r["reindex_score"] if sh else r["reindex_score"][i]
                    assert np.array_equal(rs[:len(ref)], ref), (step, b, l, i)
            for t in range(T):
                check_attention(eng.out[l, b, t].cpu().numpy(), eng.lse[l, b, t].cpu().numpy(),
                                r["out"][t], r["lse"][t],
                                "step %d seq %d layer %d token %d" % (step, b, l, t))
        _say("  checked step", step, "seq", b, "L", lens[b])


def run_block_workload(name, n_steps, seqs=None, **scale):
    wl = W.WORKLOADS[name].scaled(**scale) if scale else W.WORKLOADS[name]
    _say("workload", wl.name, "B", wl.B, "layers", wl.n_layers, "block", wl.block,
         "shared" if wl.block_shared else "per-token")
    eng = pipeline.Engine(W.Case(wl, 0, DEV), DEV)
    keys_np = eng.keys.cpu().numpy()
    cpu_case = W.Case(wl, 0, "cpu")
    for step in range(n_steps):
        eng.run_step(eng.step_inputs(step))
        torch.cuda.synchronize()
        check_engine_block(eng, cpu_case, step, seqs if seqs is not None else range(wl.B),
                           keys_np)
    return eng


@pytest.mark.parametrize("name", ["ctx_1m_block5", "ctx_1m_block5_shared"])
def test_workload_ctx_1m_block5(name):
    eng = run_block_workload(name, 1)
    out1 = eng.out.clone()
    eng.run_step(eng.step_inputs(0))
    torch.cuda.synchronize()
    assert torch.equal(out1, eng.out)


@pytest.mark.parametrize("name", ["batch8_256k_block5", "batch8_256k_block5_shared"])
def test_workload_batch_block5_appends(name):
    """Two verify steps, each appending its five tokens first, on a
    shortened batch (ragged lengths around the window)."""
    run_block_workload(name, 2, None, B=3, L=None, len_range=(130, 40000), steps=2)


# ---------------------------------------------------------------------------
# long blocks: chunked prefill indexing
# ---------------------------------------------------------------------------

def test_index_full_block_long_per_token():
    """100 tokens per sequence (four grid rows of 32 tokens, the last partial;
    chunks of 8 with a partial last chunk), ragged lengths."""
    lens = [5000, 1300, 3000]
    keys, row_off, q, w = _block_case(11, lens, 100, H=48)
    check_full_block(keys, row_off, lens, q, w, 128, 700, 40, False, "T=100")


def test_index_full_block_long_shared():
    """A shared list over 20 tokens (three chunks of 8 in one grid row)."""
    lens = [9000, 2500]
    keys, row_off, q, w = _block_case(12, lens, 20)
    check_full_block(keys, row_off, lens, q, w, 128, 1000, 64, True, "T=20 shared")


def test_workload_prefill_chunk_sampled():
    """prefill_128k_chunk256 at full size: 256 per-token pools and selections
    in one call, sampled tokens checked against the oracle (pool, scores,
    selection and attention), every token's pool length and list order
    checked."""
    wl = W.WORKLOADS["prefill_128k_chunk256"]
    T = wl.block
    eng = pipeline.Engine(W.Case(wl, 0, DEV), DEV)
    eng.run_step(eng.step_inputs(0))
    torch.cuda.synchronize()
    keys_np = eng.keys.cpu().numpy()
    case = W.Case(wl, 0, "cpu")
    L = case.lengths_at(0)[0]
    Ls = oracle.block_lengths(L, T)
    plen = eng.pool_len.cpu().numpy()
    assert plen.tolist() == [min(wl.P, x - wl.window) for x in Ls]
    pools = eng.pool_pos.cpu().numpy()
    for t in range(T):
        p = pools[t, :plen[t]]
        assert (np.diff(p) > 0).all() and p[-1] < Ls[t] - wl.window
    for t in (0, 1, 100, 255):
        q = case.index_q(0, 0, 0, t).numpy()
        w = case.index_w(0, 0, 0, t).numpy()
        rp, rs = oracle.index_full(keys_np, 0, Ls[t], q, w, wl.window, wl.P)
        assert np.array_equal(pools[t, :plen[t]], rp), t
        assert np.array_equal(eng.pool_score[t].cpu().numpy()[:plen[t]], rs), t
        sel, _ = oracle.select_topk(rs, rp, wl.k)
        assert int(eng.sel_len[0, t]) == len(sel), t
        assert np.array_equal(eng.sel_pos[0, t].cpu().numpy()[:len(sel)], sel), t
        S = oracle.attention_positions(Ls[t], sel, wl.window)
        codes, scales = oracle.fp4_quantize(u16(case.kv_bf16(0, 0, S)))
        ro, rl = oracle.attention(u16(case.attn_q(0, 0, 0, t)), codes, scales, wl.sm_scale)
        check_attention(eng.out[0, 0, t].cpu().numpy(), eng.lse[0, 0, t].cpu().numpy(), ro, rl,
                        "prefill token %d" % t)
        _say("  checked prefill token", t)


def test_index_full_block_long_batch():
    """600 per-token lists per sequence (the lists' states written by each
    sequence's first tile, two per thread); the shorter sequences' first
    tokens rank nothing (700: tokens 0-26, 600: tokens 0-127)."""
    lens = [3000, 2500, 700, 600]
    keys, row_off, q, w = _block_case(13, lens, 600, H=16)
    check_full_block(keys, row_off, lens, q, w, 128, 500, 50, False, "B=3 T=600")


def test_index_full_block_many_tiles():
    """200 per-token lists over a 90,000-position context: 19,200 tiles, so
    the gather and write kernels take four tiles per workgroup; every list
    checked in full."""
    lens = [90000]
    keys, row_off, q, w = _block_case(14, lens, 200, H=16)
    check_full_block(keys, row_off, lens, q, w, 128, 3000, 100, False, "T=200 many tiles")
