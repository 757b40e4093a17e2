"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Bar: bit-exact pool / selection / scores / FP4 bytes;
attention within 1e-3 * max|out| per (sequence, layer) and lse within
1e-3 + 1e-6 |lse| (a few fp32 spacings once |lse| is large)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from decode_kv_amd import csa2
from decode_kv_amd import inputs as I
from decode_kv_amd import pipeline
from decode_kv_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_attention(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    m = np.abs(out_ref).max()
    err = np.abs(out_gpu - out_ref).max()
    assert err <= 1e-3 * m, "%s: max err %.3g vs 1e-3*max|out| = %.3g" % (what, err, 1e-3 * m)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), what
    if fin.any():
        # 1e-3 absolute, plus a few fp32 spacings (2^-23 |lse|) for large |lse|
        tol = 1e-3 + 1e-6 * np.abs(lse_ref[fin])
        assert (np.abs(lse_gpu[fin] - lse_ref[fin]) <= tol).all(), what


# ---------------------------------------------------------------------------
# generator agreement (inputs for both sides)
# ---------------------------------------------------------------------------

def test_generator_cpu_gpu_agree():
    key = I.stream_key(5, 6)
    a = I.bf16_normal(key, 123, 100000, "cpu")
    b = I.bf16_normal(key, 123, 100000, DEV).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = I.int8_normal(key, 0, 100000, 30.0, "cpu")
    d = I.int8_normal(key, 0, 100000, 30.0, DEV).cpu()
    assert torch.equal(c, d)
    case_c = W.Case(W.WORKLOADS["ragged32_1m"], 0, "cpu")
    case_g = W.Case(W.WORKLOADS["ragged32_1m"], 0, DEV)
    assert case_c.lengths == case_g.lengths
    assert torch.equal(u16_t(case_c.kv_bf16(3, 5, [0, 77, 99999])),
                       u16_t(case_g.kv_bf16(3, 5, [0, 77, 99999]).cpu()))
    assert torch.equal(case_c.index_q(2, 4, 7), case_g.index_q(2, 4, 7).cpu())


def u16_t(t):
    return t.view(torch.int16)


# ---------------------------------------------------------------------------
# csa2_kv_append_fp4
# ---------------------------------------------------------------------------

def _finite_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_kv_append_bitexact():
    rng = np.random.default_rng(0)
    rows = []
    allv = _finite_bf16_patterns()
    rng.shuffle(allv)
    n = len(allv) // 512 * 512
    rows.append(allv[:n].reshape(-1, 512))
    for s in [-127, -125, -40, -3, 0, 7, 60, 125]:         # anchored blocks: fixed scale
        anchor = np.uint16((np.array([2.0 ** (s + 2)], np.float32).view(np.uint32) >> 16)[0])
        vals = oracle.bf16_to_f64(allv)
        ok = allv[np.abs(vals) < 2.0 ** (s + 3)]
        m = len(ok) // 31 * 31
        blk = np.zeros((m // 31, 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = ok[:m].reshape(-1, 31)
        nb = len(blk) // 16 * 16
        rows.append(blk[:nb].reshape(-1, 512))
    g = (rng.standard_normal((300, 512)) * 2.0 ** rng.integers(-30, 30, size=(300, 1)))
    rows.append((g.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    z = np.zeros((4, 512), np.uint16)
    z[1, ::3] = 0x8000
    z[2] = rng.integers(0, 128, size=512)                   # subnormals only
    z[3] = rng.integers(0, 128, size=512) | 0x8000
    rows.append(z)
    x = np.concatenate(rows)
    n = x.shape[0]
    _say("append rows", n)
    perm = rng.permutation(n + 17)[:n]
    dst = torch.tensor(perm, dtype=torch.int64, device=DEV)
    kv = torch.full((n + 17, 256), 0xEE, dtype=torch.uint8, device=DEV)
    sc = torch.full((n + 17, 16), 0xEE, dtype=torch.uint8, device=DEV)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    csa2.kv_append_fp4(xt, dst, kv, sc)
    torch.cuda.synchronize()
    codes_ref, sc_ref = oracle.fp4_quantize(x)
    assert np.array_equal(kv.cpu().numpy()[perm], codes_ref)
    assert np.array_equal(sc.cpu().numpy()[perm], sc_ref)
    untouched = np.setdiff1d(np.arange(n + 17), perm)
    assert (kv.cpu().numpy()[untouched] == 0xEE).all()


def test_kv_append_wide_rows():
    rng = np.random.default_rng(1)
    for D in [32, 96, 1024]:
        x = (rng.standard_normal((7, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        xt = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
        kv = torch.zeros((7, D // 2), dtype=torch.uint8, device=DEV)
        sc = torch.zeros((7, D // 32), dtype=torch.uint8, device=DEV)
        csa2.kv_append_fp4(xt, torch.arange(7, device=DEV), kv, sc)
        c, s = oracle.fp4_quantize(x)
        assert np.array_equal(kv.cpu().numpy(), c) and np.array_equal(sc.cpu().numpy(), s)


@pytest.mark.parametrize("D,nl", [(512, 3), (96, 3), (512, 20), (1024, 40)])
def test_append_token_bitexact(D, nl):
    """Three decode-step appends into a batch with ragged lengths (0 to 1,000,
    gaps between the sequences' rows), 3 to 40 layers (a wave of the kernel
    takes one, two or three of them): every layer's FP4 row and the index key
    land at row_off[b] + len[b], quantised exactly as the oracle does, nothing
    else changes, and each length advances by one per call."""
    rng = np.random.default_rng(41 + D + nl)
    B = 5
    lens0 = [0, 7, 129, 1000, 3]
    caps = [L + 4 for L in lens0]
    row_off, cur = [], 0
    for c in caps:
        cur += 2
        row_off.append(cur)
        cur += c
    rows = cur + 2
    kv = torch.full((nl, rows, D // 2), 0xEE, dtype=torch.uint8, device=DEV)
    sc = torch.full((nl, rows, D // 32), 0xEE, dtype=torch.uint8, device=DEV)
    keys = torch.full((rows, 64), 85, dtype=torch.int8, device=DEV)
    lens = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    ro = torch.tensor(row_off, dtype=torch.int64, device=DEV)
    want_kv, want_sc, want_keys = kv.cpu().numpy(), sc.cpu().numpy(), keys.cpu().numpy()
    for step in range(3):
        g = rng.standard_normal((nl, B, D)) * 2.0 ** rng.integers(-40, 40, size=(nl, B, 1))
        x = (g.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        kr = rng.integers(-127, 128, size=(B, 64)).astype(np.int8)
        csa2.append_token(torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16),
                          torch.from_numpy(kr).to(DEV), ro, lens, kv, sc, keys)
        codes, scales = oracle.fp4_quantize(x.reshape(nl * B, D))
        for b in range(B):
            r = row_off[b] + lens0[b] + step
            want_keys[r] = kr[b]
            for l in range(nl):
                want_kv[l, r] = codes[l * B + b]
                want_sc[l, r] = scales[l * B + b]
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), np.array(lens0) + 3)
    assert np.array_equal(keys.cpu().numpy(), want_keys)
    assert np.array_equal(kv.cpu().numpy(), want_kv)
    assert np.array_equal(sc.cpu().numpy(), want_sc)


# ---------------------------------------------------------------------------
# csa2_index_full
# ---------------------------------------------------------------------------

def run_full(keys_np, row_off, lens, q_np, w_np, window, P, k=0):
    B = len(lens)
    keys = torch.from_numpy(keys_np).to(DEV)
    ro = torch.tensor(row_off, dtype=torch.int64, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(w_np)).to(DEV)
    pos = torch.full((B, P), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    scr = torch.full((B, P), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    plen = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    sel = torch.full((B, max(k, 1)), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    slen = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    max_len, total_len = max(lens + [0]), keys_np.shape[0]
    ws = csa2.workspace(csa2.workspace_bytes(csa2.OP_INDEX_FULL, B, max_len, total_len, q.shape[1],
                                             P, k))
    csa2.index_full(q, w, keys, ro, ln, max_len, total_len, window, P, pos, scr, plen, ws,
                    k=k, sel_pos=sel if k else None, sel_len=slen if k else None)
    torch.cuda.synchronize()
    return (pos.cpu().numpy(), scr.cpu().numpy(), plen.cpu().numpy(), sel.cpu().numpy(),
            slen.cpu().numpy())


def check_full(keys_np, row_off, lens, q_np, w_np, window, P, what="", k=None):
    """Pool (and, for k > 0, the Full layer's own top k, default P // 3 + 1)
    against the oracle: the selection must be the oracle's top k of the
    oracle's pool."""
    if k is None:
        k = P // 3 + 1
    pos, scr, plen, sel, slen = run_full(keys_np, row_off, lens, q_np, w_np, window, P, k)
    for b, L in enumerate(lens):
        rp, rs = oracle.index_full(keys_np, row_off[b], L, q_np[b], w_np[b], window, P)
        n = len(rp)
        assert plen[b] == n, (what, b)
        assert np.array_equal(pos[b, :n], rp), (what, b)
        assert np.array_equal(scr[b, :n], rs), (what, b)
        assert (pos[b, n:] == -1).all() and (scr[b, n:] == -1).all(), (what, b)
        if k:
            ref, _ = oracle.select_topk(rs, rp, k)
            m = len(ref)
            assert slen[b] == m, (what, b, "selection")
            assert np.array_equal(sel[b, :m], ref), (what, b, "selection")
            assert (sel[b, m:k] == -1).all(), (what, b, "selection")
        else:
            assert (slen == -9).all() and (sel == 0x5A5A5A5A).all(), (what, "k = 0 wrote")


@pytest.mark.parametrize("seed", range(40))
def test_index_full_tiny_seeds(seed):
    case = W.Case(W.WORKLOADS["tiny_4k"], seed, "cpu")
    keys = case.keys_all().numpy()
    q, w = case.index_qw_batch(0, 0)
    k = [0, 64, 1, 1024][seed % 4]                   # 0: the pool alone; 1024: k = P
    check_full(keys, list(case.row_off), case.lengths, q.numpy(), w.numpy(), 128, 1024,
               "tiny seed %d" % seed, k=k)


def test_index_full_tie_adversarial():
    rng = np.random.default_rng(7)
    L, W_, P = 9000, 128, 1024
    keys = rng.integers(-127, 128, size=(L, 64)).astype(np.int8)
    q = rng.integers(-127, 128, size=(1, 64, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=(1, 64)).astype(np.int8)
    check_full(keys, [0], [L], np.zeros_like(q), w, W_, P, "q=0")         # all scores 0
    check_full(keys, [0], [L], q, np.zeros_like(w), W_, P, "w=0")
    same = np.tile(keys[:1], (L, 1))
    check_full(same, [0], [L], q, w, W_, P, "identical keys")
    two = np.where(rng.random((L, 1)) < 0.5, keys[:1], keys[1:2]).astype(np.int8)
    check_full(two, [0], [L], q, w, W_, P, "two distinct keys")
    few = keys[rng.integers(0, 40, size=L)]
    check_full(few, [0], [L], q, w, W_, P, "40 distinct keys")
    onehot = np.zeros_like(q)
    onehot[0, 0, 0] = 1
    w1 = np.zeros_like(w)
    w1[0, 0] = 1
    check_full(keys, [0], [L], onehot, w1, W_, P, "scores = relu(K[:,0])")


def test_index_full_clustered_scores():
    """Many distinct scores inside one second-level sub-bin, so the threshold
    needs further refinement passes before exact ranking."""
    rng = np.random.default_rng(5)
    L, W_ = 9000, 128
    keys = np.zeros((L, 64), dtype=np.int8)
    keys[:, 0] = 50
    hot = rng.choice(L - W_, 1000, replace=False)
    keys[hot, 0] = 127
    q = np.zeros((1, 64, 64), dtype=np.int8)
    q[0, 1:, 0] = 127
    q[0, 0, 1] = 1
    w = np.full((1, 64), 15, dtype=np.int8)
    w[0, 0] = 1
    # score = 120015 * k0 + relu(k1): 1,000 scores within 64 of each other
    keys[:, 1] = rng.integers(0, 64, size=L)
    check_full(keys, [0], [L], q, w, W_, 700, "64 close values")
    keys[:, 1] = rng.integers(0, 2, size=L)
    check_full(keys, [0], [L], q, w, W_, 700, "two close values, many ties")
    keys[:, 1] = rng.integers(0, 300, size=L)
    check_full(keys, [0], [L], q, w, W_, 999, "300 close values")


def test_index_full_crowded_sub_bin():
    """More than 1,024 candidates inside the second-level sub-bin, spread over
    64 values: the threshold takes a further 12-bit pass over the candidates
    (most tiles hold far more than 16 of them) before its last digits."""
    rng = np.random.default_rng(9)
    L, W_ = 20000, 128
    keys = np.zeros((L, 64), dtype=np.int8)
    keys[:, 0] = 50
    hot = rng.choice(L - W_, 5000, replace=False)
    keys[hot, 0] = 127
    keys[:, 1] = rng.integers(0, 64, size=L)
    q = np.zeros((1, 64, 64), dtype=np.int8)
    q[0, 1:, 0] = 127
    q[0, 0, 1] = 1
    w = np.full((1, 64), 15, dtype=np.int8)
    w[0, 0] = 1
    for P in [4000, 2500, 4999]:
        check_full(keys, [0], [L], q, w, W_, P, "5,000 hot over 64 values, P %d" % P)


def test_index_full_skewed_candidates():
    """Candidates of the threshold bin crowded into a few tiles (recent
    positions), and more of them than the threshold kernel's flat list holds
    (its per-tile walk), for the pool and the selection."""
    rng = np.random.default_rng(21)
    L, W_ = 20000, 128
    keys = np.zeros((L, 64), dtype=np.int8)
    keys[:, 0] = 50
    hot = L - W_ - 1 - rng.choice(900, 700, replace=False)       # 700 hot in the last tile
    keys[hot, 0] = 127
    keys[:, 1] = rng.integers(0, 64, size=L)
    q = np.zeros((1, 64, 64), dtype=np.int8)
    q[0, 1:, 0] = 127
    q[0, 0, 1] = 1
    w = np.full((1, 64), 15, dtype=np.int8)
    w[0, 0] = 1
    for P, k in [(4000, 512), (650, 100), (700, 700)]:
        check_full(keys, [0], [L], q, w, W_, P, "700 hot in one tile, P %d k %d" % (P, k), k=k)
    L2 = 40000
    keys2 = np.zeros((L2, 64), dtype=np.int8)
    keys2[:, 0] = 127
    keys2[:, 1] = rng.integers(0, 64, size=L2)
    keys2[rng.choice(L2, 5000, replace=False), 0] = 50
    for P, k in [(10000, 512), (16384, 9000)]:
        check_full(keys2, [0], [L2], q, w, W_, P, "35,000 in one bin, P %d k %d" % (P, k), k=k)


def test_index_score_matches_oracle():
    rng = np.random.default_rng(13)
    lens = [0, 1, 1023, 1024, 1025, 70001, 3000]
    row_off, cur = [], 0
    for L in lens:
        cur += 3
        row_off.append(cur)
        cur += L
    keys_np = rng.integers(-127, 128, size=(cur, 64)).astype(np.int8)
    B, H = len(lens), 64
    q_np = rng.integers(-127, 128, size=(B, H, 64)).astype(np.int8)
    w_np = rng.integers(0, 16, size=(B, H)).astype(np.int8)
    keys = torch.from_numpy(keys_np).to(DEV)
    ro = torch.tensor(row_off, dtype=torch.int64, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = torch.from_numpy(q_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    max_len = max(lens)
    ws = csa2.workspace(csa2.workspace_bytes(csa2.OP_INDEX_FULL, B, max_len, cur, H, 1))
    for window in [0, 128]:
        out = torch.full((B, max_len), -7, dtype=torch.int32, device=DEV)
        csa2.index_score(q, w, keys, ro, ln, max_len, cur, window, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for b, L in enumerate(lens):
            E = max(L - window, 0)
            ref = oracle.index_scores(keys_np, row_off[b] + np.arange(E), q_np[b], w_np[b])
            assert np.array_equal(got[b, :E], ref), (window, b)
            assert (got[b, E:] == -7).all(), (window, b)


def test_index_full_ragged_batch_and_edges():
    rng = np.random.default_rng(11)
    lens = [0, 100, 128, 129, 1152, 1153, 2048 * 3 + 128 + 17, 70001, 5000]
    gaps = [0, 3, 0, 64, 1, 0, 5, 2, 9]
    row_off, cur = [], 0
    for L, g in zip(lens, gaps):
        cur += g
        row_off.append(cur)
        cur += L
    keys = rng.integers(-127, 128, size=(cur + 5, 64)).astype(np.int8)
    B = len(lens)
    for H in [64, 4, 17, 40]:
        q = rng.integers(-127, 128, size=(B, H, 64)).astype(np.int8)
        w = rng.integers(0, 16, size=(B, H)).astype(np.int8)
        check_full(keys, row_off, lens, q, w, 128, 1024, "ragged H=%d" % H)
    q = rng.integers(-127, 128, size=(B, 64, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=(B, 64)).astype(np.int8)
    check_full(keys, row_off, lens, q, w, 0, 1, "window 0, P 1")
    check_full(keys, row_off, lens, q, w, 128, 16384, "P 16384", k=512)
    check_full(keys, row_off, lens, q, w, 128, 16384, "P 16384, pool only", k=0)


def test_index_full_long_sequences():
    """Sequences longer than 1,024 tiles, up to the 8,388,608-position maximum:
    the threshold kernel gives each thread several tiles (later rounds hold
    every candidate in its list, their starts and offsets span rounds).  Four
    index heads keep the oracle quick; 600 high keys just before the window
    crowd the selection's threshold bin into a few tiles."""
    rng = np.random.default_rng(23)
    lens = [2_500_017, 8_388_608, 1_500]
    row_off, cur = [], 0
    for L in lens:
        row_off.append(cur)
        cur += L
    keys = rng.integers(-127, 128, size=(cur, 64), dtype=np.int8)
    q = rng.integers(-127, 128, size=(len(lens), 4, 64), dtype=np.int8)
    w = rng.integers(0, 16, size=(len(lens), 4), dtype=np.int8)
    for b, L in enumerate(lens):
        if L > 10_000:
            hot = row_off[b] + L - 128 - 1 - rng.choice(3000, 600, replace=False)
            keys[hot] = np.clip(q[b, 0].astype(np.int32) + rng.integers(-3, 4, size=(600, 64)),
                                -127, 127).astype(np.int8)
    _say("long sequences", lens)
    check_full(keys, row_off, lens, q, w, 128, 16384, "long sequences, k 512", k=512)


def test_index_full_long_crowded():
    """3,000,000 positions (three rounds of tiles per threshold thread) with
    ~600,000 scores inside one first-level bin: far more candidates than the
    threshold's LDS list holds, so every pass walks the tiles from global
    memory."""
    rng = np.random.default_rng(29)
    L, W_ = 3_000_000, 128
    keys = np.zeros((L, 64), dtype=np.int8)
    keys[:, 0] = 50
    keys[rng.random(L) < 0.2, 0] = 127
    keys[:, 1] = rng.integers(0, 64, size=L)
    q = np.zeros((1, 4, 64), dtype=np.int8)
    q[0, 1:, 0] = 127
    q[0, 0, 1] = 1
    w = np.full((1, 4), 15, dtype=np.int8)
    w[0, 0] = 1
    # score = 5,715 * k0 + k1: 64 distinct values inside the hot bin
    check_full(keys, [0], [L], q, w, W_, 16384, "3M, 600K in one bin, k 512", k=512)


def test_index_full_maximum_batch():
    """4,096 sequences (the batch limit): every scoring thread maps eight of
    them to tiles; lengths 0 .. 2,600 so that some sequences have no eligible
    position and some span three tiles."""
    rng = np.random.default_rng(31)
    B = 4096
    lens = [int(x) for x in rng.integers(0, 2600, size=B)]
    lens[0], lens[1], lens[-1] = 0, 129, 2599
    row_off, cur = [], 0
    for L in lens:
        row_off.append(cur)
        cur += L
    keys = rng.integers(-127, 128, size=(cur, 64), dtype=np.int8)
    q = rng.integers(-127, 128, size=(B, 4, 64), dtype=np.int8)
    w = rng.integers(0, 16, size=(B, 4), dtype=np.int8)
    check_full(keys, row_off, lens, q, w, 128, 600, "4,096 sequences", k=100)


def test_index_full_extreme_scores():
    """Maximal scores (64 heads x 15 x 64 x 127^2) stay exact in int32."""
    L = 3000
    keys = np.full((L, 64), 127, dtype=np.int8)
    keys[::7] = -127
    keys[5::11, :3] = 0
    q = np.full((1, 64, 64), 127, dtype=np.int8)
    w = np.full((1, 64), 15, dtype=np.int8)
    check_full(keys, [0], [L], q, w, 128, 700, "extreme")


# ---------------------------------------------------------------------------
# csa2_index_reindex and csa2_select_topk
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,P", [(64, 16384), (4, 1000), (17, 3000), (33, 700), (48, 16384)])
def test_index_reindex_matches_oracle(H, P):
    """Every head-block count of the scoring instance (1 to 4 blocks of 16
    heads, the last one partly padded) and pools that end inside a
    workgroup's 256 candidates."""
    rng = np.random.default_rng(3 + H)
    B = 3
    lens = [200000, 5000, 130]
    row_off = [0, 200000, 205000]
    keys = rng.integers(-127, 128, size=(sum(lens), 64)).astype(np.int8)
    cand_len = [P, min(P, 4872), 2]
    cand = np.full((B, P), -1, dtype=np.int32)
    for b in range(B):
        cand[b, :cand_len[b]] = np.sort(rng.choice(max(lens[b] - 128, 2), cand_len[b], replace=False))
    q = rng.integers(-127, 128, size=(B, H, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=(B, H)).astype(np.int8)
    score = torch.full((B, P), 0x7777, dtype=torch.int32, device=DEV)
    csa2.index_reindex(torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV),
                       torch.from_numpy(keys).to(DEV),
                       torch.tensor(row_off, dtype=torch.int64, device=DEV),
                       torch.from_numpy(cand).to(DEV),
                       torch.tensor(cand_len, dtype=torch.int32, device=DEV), score)
    got = score.cpu().numpy()
    for b in range(B):
        n = cand_len[b]
        ref = oracle.index_reindex(keys, row_off[b], cand[b, :n], q[b], w[b])
        assert np.array_equal(got[b, :n], ref)
        assert (got[b, n:] == -1).all()


def test_select_topk_short_rows():
    """Rows of P = 1,000 candidates (fewer than the workgroup's threads), full,
    partial, short and empty lists, k up to P."""
    rng = np.random.default_rng(77)
    B, P = 4, 1000
    cand_len = [1000, 700, 37, 0]
    score = rng.integers(0, 5000, size=(B, P)).astype(np.int32)
    cand = np.zeros((B, P), dtype=np.int32)
    for b in range(B):
        cand[b] = np.sort(rng.choice(1_000_000, P, replace=False))
    for k in [1, 37, 500, 1000]:
        sel = torch.full((B, k), 0x3333, dtype=torch.int32, device=DEV)
        sl = torch.full((B,), -5, dtype=torch.int32, device=DEV)
        csa2.select_topk(torch.from_numpy(score).to(DEV), torch.from_numpy(cand).to(DEV),
                         torch.tensor(cand_len, dtype=torch.int32, device=DEV), k, sel, sl)
        got, gl = sel.cpu().numpy(), sl.cpu().numpy()
        for b in range(B):
            n = cand_len[b]
            ref, _ = oracle.topk(score[b, :n], cand[b, :n], k)
            assert gl[b] == len(ref), (k, b)
            assert np.array_equal(got[b, :len(ref)], ref), (k, b)
            assert (got[b, len(ref):] == -1).all(), (k, b)


@pytest.mark.parametrize("span", [3, 50, 100000, 1 << 30])
def test_select_topk_matches_oracle(span):
    rng = np.random.default_rng(span % 1000)
    B, P = 4, 16384
    cand_len = [16384, 9000, 512, 37]
    score = rng.integers(0, span, size=(B, P)).astype(np.int32)
    cand = np.zeros((B, P), dtype=np.int32)
    for b in range(B):
        cand[b] = np.sort(rng.choice(10_000_000, P, replace=False))
    for k in [1, 64, 512, 16384]:
        sel = torch.full((B, k), 0x3333, dtype=torch.int32, device=DEV)
        sl = torch.zeros(B, dtype=torch.int32, device=DEV)
        csa2.select_topk(torch.from_numpy(score).to(DEV), torch.from_numpy(cand).to(DEV),
                         torch.tensor(cand_len, dtype=torch.int32, device=DEV), k, sel, sl)
        got, gl = sel.cpu().numpy(), sl.cpu().numpy()
        for b in range(B):
            n = cand_len[b]
            ref, _ = oracle.topk(score[b, :n], cand[b, :n], k)
            assert gl[b] == len(ref)
            assert np.array_equal(got[b, :len(ref)], ref), (span, k, b)
            assert (got[b, len(ref):] == -1).all()


@pytest.mark.parametrize("top_span", [40, 2000, 1 << 20])
def test_select_topk_clustered(top_span):
    """A cluster of 700 scores near 2^20 above a low background: the bin that
    holds the 512th score then has far more than 256 entries, so the select
    narrows it with further digits (to one value with ties when top_span is
    small); the shorter lists keep the cluster and drop the background."""
    rng = np.random.default_rng(top_span)
    B, P = 3, 16384
    cand_len = [16384, 5000, 1100]
    score = rng.integers(0, 1000, size=(B, P)).astype(np.int32)
    cand = np.zeros((B, P), dtype=np.int32)
    for b in range(B):
        hot = rng.choice(cand_len[b], 700, replace=False)
        score[b, hot] = (1 << 20) + rng.integers(0, top_span, size=700)
        cand[b] = np.sort(rng.choice(10_000_000, P, replace=False))
    for k in [1, 300, 512, 699, 700, 1024]:
        sel = torch.full((B, k), 0x3333, dtype=torch.int32, device=DEV)
        sl = torch.zeros(B, dtype=torch.int32, device=DEV)
        csa2.select_topk(torch.from_numpy(score).to(DEV), torch.from_numpy(cand).to(DEV),
                         torch.tensor(cand_len, dtype=torch.int32, device=DEV), k, sel, sl)
        got, gl = sel.cpu().numpy(), sl.cpu().numpy()
        for b in range(B):
            n = cand_len[b]
            ref, _ = oracle.topk(score[b, :n], cand[b, :n], k)
            assert gl[b] == len(ref)
            assert np.array_equal(got[b, :len(ref)], ref), (top_span, k, b)
            assert (got[b, len(ref):] == -1).all()


# ---------------------------------------------------------------------------
# csa2_sparse_attn_decode
# ---------------------------------------------------------------------------

def run_attention(codes, scales, row_off, lens, sel, sel_len, q_bits, k, window):
    """Two calls on one workspace: the second (into fresh NaN outputs) must be
    bit-identical (nothing carries over between calls)."""
    B, Hq, D = q_bits.shape
    qt = torch.from_numpy(q_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    ws = csa2.workspace(csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, B, 0, 0, 0, 0, k, Hq, D, window))
    args = (torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
            torch.tensor(row_off, dtype=torch.int64, device=DEV),
            torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens + [0]),
            torch.from_numpy(sel).to(DEV), torch.tensor(sel_len, dtype=torch.int32, device=DEV),
            k, window, 1 / math.sqrt(D))
    res = []
    for _ in range(2):
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        csa2.sparse_attn_decode(qt, *args, out, lse, ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0], equal_nan=True)
    assert np.array_equal(res[0][1], res[1][1], equal_nan=True)
    return res[0]


def attention_case(seed, lens, k, Hq, scale_lo=118, scale_hi=130, window=128, q_exp=None):
    """Random FP4 rows (every code, scale bytes uniform in [scale_lo, scale_hi])
    and bf16 queries: N(0,1), or with q_exp, magnitudes in [0.25, 4) times
    2^q_exp (all normal bf16), so that caches with huge scales keep every
    score finite in fp32."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    row_off = list(np.cumsum([0] + lens[:-1]))
    n = max(1, sum(lens))
    codes_t, scales_t = W.raw_fp4_rows(seed, n, 512, scale_lo, scale_hi)
    codes, scales = codes_t.numpy(), scales_t.numpy()
    sel = np.full((B, k), -1, dtype=np.int32)
    sel_len = []
    for b, L in enumerate(lens):
        E = max(0, L - window)
        m = min(k, E, int(rng.integers(0, k + 1)) if seed % 3 == 0 else k)
        if m:
            sel[b, :m] = np.sort(rng.choice(E, m, replace=False))
        sel_len.append(m)
    qf = rng.standard_normal((B, Hq, 512))
    if q_exp is not None:
        qf = np.sign(qf) * np.clip(np.abs(qf), 0.25, 3.99) * 2.0 ** q_exp
    q = (qf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out, lse = run_attention(codes, scales, row_off, lens, sel, sel_len, q, k, window)
    for b, L in enumerate(lens):
        S = oracle.attention_positions(L, sel[b, :sel_len[b]], window)
        rows = row_off[b] + S
        ro, rl = oracle.attention(q[b], codes[rows], scales[rows], 1 / math.sqrt(512))
        check_attention(out[b], lse[b], ro, rl, "seed %d b %d L %d" % (seed, b, L))


@pytest.mark.parametrize("seed", range(6))
def test_attention_random_fp4(seed):
    attention_case(seed, [4096, 70000, 1000, 640, 129], 512, 64)


def test_attention_small_heads_and_short_contexts():
    attention_case(10, [4096], 64, 16)
    attention_case(11, [50, 128, 129, 0, 300], 64, 16)
    attention_case(12, [5000] * 3, 64, 128)
    attention_case(13, [100000], 512, 64, window=0)
    attention_case(14, [3000] * 32, 512, 64)         # 640 workgroups: the wide tile layout


def test_attention_many_splits():
    attention_case(15, [40000], 8192, 64)           # 260 tiles over 65 splits (wide layout)
    attention_case(16, [20000, 300, 9000], 2048, 32)


def test_attention_maximum_rows_and_many_pairs():
    attention_case(17, [20000], 16384 - 128, 16)    # k + window = 16,384: 512 tiles, 128 splits
    attention_case(18, [700] * 12, 256, 64)         # 48 (sequence, head group) pairs > 8
    attention_case(19, [int(x) for x in np.random.default_rng(19).integers(0, 900, size=200)],
                   128, 16)                          # 200 sequences, some empty (wide layout)


def test_attention_batched_shapes():
    """Batches placed sequence-major (8 sequences and more): 65 splits per
    sequence merged in chunks of 32 by the combine (8 sequences, k = 8,192),
    12 sequences of 48 heads, ragged lengths with empty sequences and
    sequences shorter than the window."""
    attention_case(30, [20000] * 8, 8192, 16)
    attention_case(31, [700] * 12, 256, 48)
    attention_case(32, [0, 50, 129, 3000, 0, 640, 12000, 77, 4096, 1], 512, 64)


def test_attention_uneven_window_and_head_groups():
    """A 300-token window with k = 100 (400 rows: a partial last tile) and 80
    query heads (five 16-head groups per sequence, an odd pair count per
    XCD); sequences shorter than the window and one with no selection."""
    attention_case(33, [5000, 900, 200, 120], 100, 80, window=300)
    attention_case(34, [3000] * 9, 100, 80, window=300)    # sequence-major placement


def test_attention_scale_ranges():
    attention_case(20, [4096, 2000], 512, 64, scale_lo=100, scale_hi=150)
    attention_case(21, [4096, 2000], 512, 64, scale_lo=1, scale_hi=1)


def test_attention_smallest_scale_byte():
    """Scale byte 0 (2^-127) on every block with non-zero codes: every value
    is at most 6 * 2^-127, many are bf16 subnormals, and the outputs are fp32
    subnormals; one sequence alone (single split) and a batch (split-K)."""
    attention_case(22, [4096, 2000], 512, 64, scale_lo=0, scale_hi=0)
    attention_case(23, [3000], 512, 64, scale_lo=0, scale_hi=2)
    attention_case(24, [2500] * 16, 512, 64, scale_lo=0, scale_hi=0)     # wide layout


def test_attention_largest_scale_bytes():
    """Scale bytes 240..252 (the largest the append produces for finite bf16):
    values up to 6 * 2^125, whose unnormalised softmax sums would overflow
    fp32; the queries are small enough that the scores stay finite."""
    attention_case(25, [4096, 2000], 512, 64, scale_lo=240, scale_hi=252, q_exp=-121)
    attention_case(26, [4096, 2000], 512, 64, scale_lo=250, scale_hi=252, q_exp=-124)
    attention_case(27, [2500] * 16, 512, 64, scale_lo=240, scale_hi=252, q_exp=-124)


def test_attention_full_scale_range():
    """Scale bytes drawn from the whole finite range 0..252 block by block, so
    the rows of one workgroup span 252 octaves."""
    attention_case(28, [4096, 2000], 512, 64, scale_lo=0, scale_hi=252, q_exp=-124)
    attention_case(29, [40000], 8192, 64, scale_lo=0, scale_hi=252, q_exp=-124)


def test_attention_empty_sequence():
    out, lse = run_attention(np.zeros((8, 256), np.uint8), np.zeros((8, 16), np.uint8), [0, 0],
                             [0, 8], np.full((2, 16), -1, np.int32), [0, 0],
                             np.ones((2, 16, 512), np.uint16), 16, 128)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(out[1]).all()


# ---------------------------------------------------------------------------
# whole decode steps through the pipeline
# ---------------------------------------------------------------------------

def check_engine_step(eng: pipeline.Engine, cpu_case: W.Case, step: int, seqs, keys_np):
    wl = eng.wl
    lens = cpu_case.lengths_at(step)
    for b in seqs:
        off = int(cpu_case.row_off[b])
        kb = keys_np[off:off + cpu_case.caps[b]]
        idx_q = {l: cpu_case.index_q(step, l, b).numpy() for l, c in enumerate(wl.pattern) if c in "FR"}
        idx_w = {l: cpu_case.index_w(step, l, b).numpy() for l, c in enumerate(wl.pattern) if c in "FR"}
        attn_q = [u16(cpu_case.attn_q(step, l, b)) for l in range(wl.n_layers)]
        res = oracle.decode_step(wl.pattern, kb, 0, lens[b], wl.window, wl.P, wl.k, idx_q, idx_w,
                                 attn_q, lambda l, S: u16(cpu_case.kv_bf16(l, b, S)), wl.sm_scale)
        pool_len = int(eng.pool_len[b])
        pool = eng.pool_pos[b].cpu().numpy()
        assert pool_len == len(res[0]["pool_pos"]), (step, b)
        assert np.array_equal(pool[:pool_len], res[0]["pool_pos"]), (step, b)
        assert np.array_equal(eng.pool_score[b].cpu().numpy()[:pool_len], res[0]["pool_score"])
        assert (pool[pool_len:] == -1).all()
        for l, r in enumerate(res):
            src = eng.selection_layer(l)
            sl = int(eng.sel_len[src, b])
            sel = eng.sel_pos[src, b].cpu().numpy()
            assert sl == len(r["sel"]), (step, b, l)
            assert np.array_equal(sel[:sl], r["sel"]), (step, b, l)
            if r["kind"] == "R":
                rs = eng.rscore[l, b].cpu().numpy()
                assert np.array_equal(rs[:pool_len], r["reindex_score"]), (step, b, l)
            check_attention(eng.out[l, b].cpu().numpy(), eng.lse[l, b].cpu().numpy(), r["out"],
                            r["lse"], "step %d seq %d layer %d" % (step, b, l))
        _say("  checked step", step, "seq", b, "L", lens[b])


def run_workload(name, steps, seqs=None, **scale):
    wl = W.WORKLOADS[name].scaled(**scale) if scale else W.WORKLOADS[name]
    _say("workload", wl.name, "B", wl.B, "layers", wl.n_layers)
    eng = pipeline.Engine(W.Case(wl, 0, DEV), DEV)
    keys_np = eng.keys.cpu().numpy()                       # generator output, before any step
    cpu_case = W.Case(wl, 0, "cpu")
    for step in range(steps):
        eng.run_step(eng.step_inputs(step))
        torch.cuda.synchronize()
        check_engine_step(eng, cpu_case, step, seqs if seqs is not None else range(wl.B), keys_np)
    return eng


def test_workload_tiny_4k():
    run_workload("tiny_4k", 1)


def test_workload_single_64k():
    run_workload("single_64k", 1)


def test_workload_batch8_256k_two_steps():
    run_workload("batch8_256k", 2)


def test_workload_ctx_1m():
    eng = run_workload("ctx_1m", 1)
    # determinism: the same step again gives identical bits
    out1, pool1 = eng.out.clone(), eng.pool_pos.clone()
    eng.run_step(eng.step_inputs(0))
    torch.cuda.synchronize()
    assert torch.equal(out1, eng.out) and torch.equal(pool1, eng.pool_pos)


def test_append_steps_side_stream_and_graph_replay():
    """Decode steps with appends run three ways give identical bits: eagerly
    on torch's current stream, eagerly on a stream that is not current (every
    call, the append included, is enqueued on the stream it is given), and as
    one captured step replayed with fresh inputs, the lengths advancing on the
    device.  The last step is also checked against the oracle."""
    wl = W.WORKLOADS["ragged32_1m"].scaled(B=4, len_range=(300, 30000), n_layers=5, steps=4)
    engs = [pipeline.Engine(W.Case(wl, 3, DEV), DEV) for _ in range(3)]
    keys_np = engs[0].keys.cpu().numpy()
    for step in range(wl.steps):
        engs[0].run_step(engs[0].step_inputs(step))
    side = torch.cuda.Stream()
    for step in range(wl.steps):
        inp = engs[1].step_inputs(step)
        side.wait_stream(torch.cuda.current_stream())
        engs[1].run_step(inp, stream=side)
        torch.cuda.current_stream().wait_stream(side)
    static = engs[2].step_inputs(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        engs[2].run_step(static)
    for step in range(wl.steps):
        pipeline.copy_inputs(static, engs[2].step_inputs(step))
        graph.replay()
    torch.cuda.synchronize()
    names = ["lens", "keys", "kv_fp4", "kv_scale", "pool_pos", "pool_score", "pool_len",
             "rscore", "sel_pos", "sel_len", "out", "lse"]
    for e in engs[1:]:
        for n in names:
            assert torch.equal(getattr(engs[0], n), getattr(e, n)), n
    assert engs[0].lens.cpu().tolist() == W.Case(wl, 3, "cpu").lengths_at(wl.steps - 1)
    check_engine_step(engs[0], W.Case(wl, 3, "cpu"), wl.steps - 1, [0, 3], keys_np)


def test_workload_ctx_1m_shared_kv():
    run_workload("ctx_1m_shared", 1)


def test_workload_ragged32_shared_kv_sampled():
    case = W.Case(W.WORKLOADS["ragged32_1m_shared"], 0, "cpu")
    order = np.argsort(case.lengths)
    run_workload("ragged32_1m_shared", 2, sorted({int(order[0]), int(order[-1]), 9}))


def test_workload_ragged32_sampled():
    case = W.Case(W.WORKLOADS["ragged32_1m"], 0, "cpu")
    order = np.argsort(case.lengths)
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 5})
    run_workload("ragged32_1m", 2, seqs)
