"""Pins of the oracle's index scores, rank order, Full / Reindex / Reuse modes
and window rule against a hand-worked example, closed forms, plain-Python
brute force and exhaustive rank counting."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    d = {"q": [], "k": []}
    with open(os.path.join(GOLDEN, "score_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag in ("q", "k"):
                d[tag].append([int(v) for v in vals])
            elif tag == "top":
                d.setdefault("top", {})[int(vals[0])] = [int(v) for v in vals[1:]]
            else:
                d[tag] = [int(v) for v in vals]
    return d


def test_hand_worked_scores_and_topk():
    d = _hand()
    q = np.array(d["q"], dtype=np.int8)
    w = np.array(d["w"], dtype=np.int8)
    keys = np.array(d["k"], dtype=np.int8)
    L, W = d["L"][0], d["window"][0]
    assert oracle.eligible_count(L, W) == 6
    pos, sc = oracle.index_full(keys, 0, L, q, w, W, 6)
    assert list(pos) == [0, 1, 2, 3, 4, 5]
    assert list(sc) == d["scores"]
    for k, want in d["top"].items():
        got, _ = oracle.select_topk(sc, pos, k)
        assert list(got) == want
        got_full, _ = oracle.index_full(keys, 0, L, q, w, W, k)
        assert list(got_full) == want


def _brute_scores(keys, rows, q, w):
    out = []
    for r in rows:
        s = 0
        for h in range(len(q)):
            dot = sum(int(a) * int(b) for a, b in zip(q[h], keys[r]))
            s += int(w[h]) * max(0, dot)
        out.append(s)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_scores_match_plain_python(seed):
    rng = np.random.default_rng(seed)
    H, dk, n = int(rng.integers(1, 9)), 64, 40
    keys = rng.integers(-127, 128, size=(n, dk)).astype(np.int8)
    q = rng.integers(-127, 128, size=(H, dk)).astype(np.int8)
    w = rng.integers(0, 16, size=H).astype(np.int8)
    rows = rng.permutation(n)[:25]
    assert list(oracle.index_scores(keys, rows, q, w)) == _brute_scores(keys, rows, q, w)


def test_score_closed_forms():
    rng = np.random.default_rng(3)
    keys = rng.integers(-127, 128, size=(300, 64)).astype(np.int8)
    rows = np.arange(300)
    H = 8
    # one-hot query on (head h, dim d) with weight only on h: s = w_h*max(0, c*K[p][d])
    for h, d, c, wh in [(0, 0, 1, 1), (3, 17, -5, 7), (7, 63, 127, 15)]:
        q = np.zeros((H, 64), dtype=np.int8)
        q[h, d] = c
        w = np.zeros(H, dtype=np.int8)
        w[h] = wh
        want = wh * np.maximum(0, c * keys[:, d].astype(np.int64))
        assert np.array_equal(oracle.index_scores(keys, rows, q, w), want)
    q = rng.integers(-127, 128, size=(H, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=H).astype(np.int8)
    assert not oracle.index_scores(keys, rows, np.zeros_like(q), w).any()
    assert not oracle.index_scores(keys, rows, q, np.zeros_like(w)).any()


def test_score_relu_and_weight_linearity():
    rng = np.random.default_rng(4)
    keys = rng.integers(-127, 128, size=(500, 64)).astype(np.int8)
    rows = np.arange(500)
    H = 16
    q = rng.integers(-127, 128, size=(H, 64)).astype(np.int8)
    w1 = rng.integers(0, 8, size=H).astype(np.int8)
    w2 = rng.integers(0, 8, size=H).astype(np.int8)
    s_pos = oracle.index_scores(keys, rows, q, w1)
    s_neg = oracle.index_scores(keys, rows, -q, w1)
    dots = keys.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(s_pos + s_neg, np.abs(dots) @ w1.astype(np.int64))
    assert np.array_equal(oracle.index_scores(keys, rows, q, w1 + w2),
                          s_pos + oracle.index_scores(keys, rows, q, w2))


def test_score_upper_bound():
    keys = np.full((2, 64), 127, dtype=np.int8)
    keys[1] = -127
    q = np.full((64, 64), 127, dtype=np.int8)
    w = np.full(64, 15, dtype=np.int8)
    s = oracle.index_scores(keys, np.arange(2), q, w)
    assert list(s) == [64 * 15 * 64 * 127 * 127, 0]
    assert s[0] == 990965760 and s[0] < 2 ** 31


def _rank_count_topk(score, pos, k):
    """p is kept iff fewer than k candidates precede it (exhaustive count)."""
    keep = []
    for i in range(len(score)):
        ahead = sum(1 for j in range(len(score))
                    if score[j] > score[i] or (score[j] == score[i] and pos[j] < pos[i]))
        if ahead < k:
            keep.append(int(pos[i]))
    return sorted(keep)


@pytest.mark.parametrize("seed", range(10))
def test_topk_equals_exhaustive_rank(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 120))
    span = int(rng.choice([3, 10, 1000]))          # small spans force many ties
    score = rng.integers(0, span, size=n)
    pos = np.sort(rng.choice(10 * n, size=n, replace=False))
    for k in [1, 2, n // 3, n - 1, n, n + 5]:
        if k < 1:
            continue
        got, gs = oracle.topk(score, pos, k)
        assert list(got) == _rank_count_topk(score, pos, k)
        order = np.lexsort((pos, -score))[:min(k, n)]
        assert list(got) == sorted(pos[order].tolist())
        lookup = dict(zip(pos.tolist(), score.tolist()))
        assert [lookup[p] for p in got] == list(gs)


def test_topk_special_orders():
    n = 50
    pos = np.arange(n)
    got, _ = oracle.topk(np.full(n, 7), pos, 10)
    assert list(got) == list(range(10))                 # all equal -> first positions
    got, _ = oracle.topk(np.arange(n)[::-1].copy(), pos, 10)
    assert list(got) == list(range(10))                 # decreasing -> first k
    got, _ = oracle.topk(np.arange(n), pos, 10)
    assert list(got) == list(range(40, 50))             # increasing -> last k


def test_duplicate_keys_lower_position_wins():
    rng = np.random.default_rng(9)
    keys = rng.integers(-20, 20, size=(400, 64)).astype(np.int8)
    keys[[50, 120, 300]] = 100                          # three identical strong keys
    q = np.full((2, 64), 3, dtype=np.int8)
    w = np.array([1, 1], dtype=np.int8)
    pos, _ = oracle.index_full(keys, 0, 400 + 128, q, w, 128, 2)
    assert list(pos) == [50, 120]


def test_full_pool_is_all_eligible_when_P_covers_E():
    rng = np.random.default_rng(5)
    L, W = 700, 128
    keys = rng.integers(-127, 128, size=(L, 64)).astype(np.int8)
    q = rng.integers(-127, 128, size=(4, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=4).astype(np.int8)
    pos, sc = oracle.index_full(keys, 0, L, q, w, W, 10_000)
    assert list(pos) == list(range(L - W))
    assert np.array_equal(sc, oracle.index_scores(keys, np.arange(L - W), q, w))


@pytest.mark.parametrize("seed", range(4))
def test_full_selection_is_global_topk(seed):
    """The pool contains the global top-k, so selecting k from the pool equals
    selecting k from every eligible position."""
    rng = np.random.default_rng(seed)
    L, W, P, k = int(rng.integers(300, 900)), 128, 120, 30
    keys = rng.integers(-127, 128, size=(L + 50, 64)).astype(np.int8)
    off = 50
    q = rng.integers(-127, 128, size=(4, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=4).astype(np.int8)
    pool, ps = oracle.index_full(keys, off, L, q, w, W, P)
    sel, _ = oracle.select_topk(ps, pool, k)
    E = L - W
    all_s = oracle.index_scores(keys, off + np.arange(E), q, w)
    assert list(sel) == _rank_count_topk(all_s, np.arange(E), k)
    assert list(pool) == _rank_count_topk(all_s, np.arange(E), P)
    assert (np.diff(pool) > 0).all() and pool.max() < E


def test_reindex_with_whole_context_equals_full():
    rng = np.random.default_rng(6)
    L, W, k = 900, 128, 40
    keys = rng.integers(-127, 128, size=(L, 64)).astype(np.int8)
    q = rng.integers(-127, 128, size=(8, 64)).astype(np.int8)
    w = rng.integers(0, 16, size=8).astype(np.int8)
    E = L - W
    pool, ps = oracle.index_full(keys, 0, L, q, w, W, E)
    rs = oracle.index_reindex(keys, 0, pool, q, w)
    assert np.array_equal(rs, ps)
    a, _ = oracle.select_topk(rs, pool, k)
    b, _ = oracle.index_full(keys, 0, L, q, w, W, k)
    assert np.array_equal(a, b)


def _distinct_sequences(rng, lens, gap=7):
    """Index keys of several sequences in one cache, each sequence drawn from
    its own range so that reading the wrong rows changes every score."""
    row_off, parts, cur = [], [], 0
    for b, L in enumerate(lens):
        pad = rng.integers(-127, 128, size=(gap, 64))
        parts.append(pad)
        cur += gap
        row_off.append(cur)
        lo = -127 + 40 * b
        parts.append(rng.integers(lo, lo + 60, size=(L, 64)))
        cur += L
    return np.concatenate(parts).astype(np.int8), row_off


def test_reindex_row_offset_matches_brute_force():
    """Reindex reads sequence b's keys at row_off[b] + position: scores of the
    pool of a sequence placed after others in the cache equal plain-Python
    scores of exactly those rows (and differ from the rows at offset 0)."""
    rng = np.random.default_rng(12)
    keys, row_off = _distinct_sequences(rng, [300, 500, 200])
    q = rng.integers(-127, 128, size=(5, 64)).astype(np.int8)
    w = rng.integers(1, 16, size=5).astype(np.int8)
    for b, L in enumerate([300, 500, 200]):
        cand = np.sort(rng.choice(L, 60, replace=False))
        got = oracle.index_reindex(keys, row_off[b], cand, q, w)
        assert list(got) == _brute_scores(keys, row_off[b] + cand, q, w)
        if b:
            assert list(got) != _brute_scores(keys, cand, q, w)


def test_decode_step_row_offset():
    """A whole decode step of a sequence stored at a non-zero row offset:
    the Full pool and selection are the exhaustive ranking of plain-Python
    scores of rows row_off + p, and each Reindex score is the plain-Python
    score of row row_off + pool position with that layer's query."""
    rng = np.random.default_rng(13)
    lens = [400, 700]
    keys, row_off = _distinct_sequences(rng, lens)
    W, P, k, H, D = 128, 90, 20, 3, 512
    b, L = 1, lens[1]
    off = row_off[b]
    qs = {l: rng.integers(-127, 128, size=(H, 64)).astype(np.int8) for l in (0, 1, 4)}
    ws = {l: rng.integers(0, 16, size=H).astype(np.int8) for l in (0, 1, 4)}
    attn_q = [np.zeros((16, D), dtype=np.uint16) for _ in range(5)]
    kv = np.zeros((L, D), dtype=np.uint16)
    res = oracle.decode_step("FRUUR", keys, off, L, W, P, k, qs, ws, attn_q,
                             lambda l, S: kv[S], 1 / math.sqrt(D))
    E = L - W
    s0 = _brute_scores(keys, off + np.arange(E), qs[0], ws[0])
    assert list(res[0]["pool_pos"]) == _rank_count_topk(s0, np.arange(E), P)
    assert list(res[0]["sel"]) == _rank_count_topk(s0, np.arange(E), k)
    pool = res[0]["pool_pos"]
    for l in (1, 4):
        want = _brute_scores(keys, off + pool, qs[l], ws[l])
        assert list(res[l]["reindex_score"]) == want
        assert list(res[l]["sel"]) == _rank_count_topk(want, pool, k)
    assert np.array_equal(res[2]["sel"], res[1]["sel"]) and np.array_equal(res[3]["sel"], res[1]["sel"])


def test_window_and_eligibility():
    for L, W in [(0, 128), (5, 128), (128, 128), (129, 128), (4096, 128), (10, 0)]:
        E = oracle.eligible_count(L, W)
        win = oracle.window_positions(L, W)
        assert E == max(0, L - W)
        assert list(win) == list(range(max(0, L - W), L))
        sel = np.arange(0, E, 3)
        S = oracle.attention_positions(L, sel, W)
        assert len(set(S.tolist())) == len(S) == len(sel) + min(W, L)
        assert not set(sel.tolist()) & set(win.tolist())
    with pytest.raises(AssertionError):
        oracle.attention_positions(300, np.array([250]), 128)


def test_layer_pattern():
    assert oracle.layer_pattern(20) == "FRUURUUURUUURUUURUUU"
    assert oracle.layer_pattern(4) == "FRUU"
    assert oracle.layer_pattern(1) == "F"
