"""Pins of the oracle's multi-token (verify block) decode step: a block of
one token is the single-token step, the pools are the exhaustive ranking of
plain-Python scores over each token's causal eligible set (per token) or of
the best score over the block (shared), a token never sees positions after
itself, and with every position selected each token's output is dense causal
softmax attention."""
import math

import numpy as np
import pytest
import scipy.special

import oracle


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _plain_scores(keys, rows, q, w):
    out = []
    for r in rows:
        s = 0
        for h in range(len(q)):
            dot = sum(int(a) * int(b) for a, b in zip(q[h], keys[r]))
            s += int(w[h]) * max(0, dot)
        out.append(s)
    return out


def _rank(score, pos, k):
    """Positions kept when p is kept iff fewer than k candidates precede it."""
    keep = []
    for i in range(len(score)):
        ahead = sum(1 for j in range(len(score))
                    if score[j] > score[i] or (score[j] == score[i] and pos[j] < pos[i]))
        if ahead < k:
            keep.append(int(pos[i]))
    return sorted(keep)


def _setup(seed, L, T, H=3, Hq=4, D=64, n_layers=4):
    rng = np.random.default_rng(seed)
    keys = rng.integers(-60, 61, size=(L, 64)).astype(np.int8)
    idx_q = {l: rng.integers(-60, 61, size=(T, H, 64)).astype(np.int8) for l in range(n_layers)}
    idx_w = {l: rng.integers(0, 16, size=(T, H)).astype(np.int8) for l in range(n_layers)}
    attn_q = [_bf16(rng.standard_normal((T, Hq, D))) for _ in range(n_layers)]
    kv = [_bf16(rng.standard_normal((L, D))) for _ in range(n_layers)]
    return keys, idx_q, idx_w, attn_q, kv


def test_block_lengths():
    assert oracle.block_lengths(10, 5) == [6, 7, 8, 9, 10]
    assert oracle.block_lengths(7, 1) == [7]


@pytest.mark.parametrize("shared", [False, True])
def test_block_of_one_is_the_single_token_step(shared):
    L, W, P, k = 700, 32, 90, 20
    keys, idx_q, idx_w, attn_q, kv = _setup(1, L, 1)
    blk = oracle.decode_block("FRUR", keys, 0, L, 1, W, P, k, idx_q, idx_w, attn_q,
                              lambda l, S: kv[l][S], 0.125, shared)
    one = oracle.decode_step("FRUR", keys, 0, L, W, P, k, {l: q[0] for l, q in idx_q.items()},
                             {l: w[0] for l, w in idx_w.items()}, [q[0] for q in attn_q],
                             lambda l, S: kv[l][S], 0.125)
    for a, b in zip(blk, one):
        sel = a["sel"] if shared else a["sel"][0]
        assert np.array_equal(sel, b["sel"])
        assert np.array_equal(a["out"][0], b["out"]) and np.array_equal(a["lse"][0], b["lse"])
    pool = blk[0]["pool_pos"] if shared else blk[0]["pool_pos"][0]
    assert np.array_equal(pool, one[0]["pool_pos"])


def test_per_token_pools_are_each_tokens_own_ranking():
    L, T, W, P = 140, 5, 16, 30
    keys, idx_q, idx_w, _, _ = _setup(2, L, T)
    res = oracle.index_full_block(keys, 0, L, T, idx_q[0], idx_w[0], W, P, shared=False)
    for t, (pos, sc) in enumerate(res):
        E = L - T + 1 + t - W                             # token t's eligible positions
        s = _plain_scores(keys, range(E), idx_q[0][t], idx_w[0][t])
        assert list(pos) == _rank(s, list(range(E)), P)
        assert list(sc) == [s[p] for p in pos]


def test_shared_pool_ranks_the_best_score_of_the_block():
    L, T, W, P = 140, 5, 16, 30
    keys, idx_q, idx_w, _, _ = _setup(3, L, T)
    pos, sc = oracle.index_full_block(keys, 0, L, T, idx_q[0], idx_w[0], W, P, shared=True)
    E0 = L - T + 1 - W                                    # eligible for every token
    per = [_plain_scores(keys, range(E0), idx_q[0][t], idx_w[0][t]) for t in range(T)]
    best = [max(per[t][p] for t in range(T)) for p in range(E0)]
    assert list(pos) == _rank(best, list(range(E0)), P)
    assert list(sc) == [best[p] for p in pos]
    cand = np.array([3, 17, 40, 41, 99])
    got = oracle.index_reindex_block(keys, 0, cand, idx_q[1], idx_w[1], shared=True)
    want = [max(_plain_scores(keys, [p], idx_q[1][t], idx_w[1][t])[0] for t in range(T)) for p in cand]
    assert list(got) == want


def test_shared_equals_per_token_when_the_tokens_agree():
    L, T, W, P = 400, 5, 16, 50
    keys, idx_q, idx_w, _, _ = _setup(4, L, T)
    q = np.repeat(idx_q[0][:1], T, axis=0)
    w = np.repeat(idx_w[0][:1], T, axis=0)
    shared = oracle.index_full_block(keys, 0, L, T, q, w, W, P, shared=True)
    per = oracle.index_full_block(keys, 0, L, T, q, w, W, P, shared=False)
    assert np.array_equal(shared[0], per[0][0]) and np.array_equal(shared[1], per[0][1])


@pytest.mark.parametrize("shared", [False, True])
def test_a_token_does_not_see_later_positions(shared):
    """Changing the FP4 row and the index key of position L_t (the first one
    token t cannot see) leaves token t unchanged and changes token t + 1, whose
    window holds it."""
    L, T, W, P, k = 600, 5, 32, 80, 25
    keys, idx_q, idx_w, attn_q, kv = _setup(5, L, T)
    t = 2
    Lt = oracle.block_lengths(L, T)[t]
    run = lambda ks, rows: oracle.decode_block("FRU", ks, 0, L, T, W, P, k, idx_q, idx_w, attn_q,
                                               lambda l, S: rows[l][S], 0.125, shared)
    base = run(keys, kv)
    keys2 = keys.copy()
    keys2[Lt] = 127 - keys2[Lt]
    kv2 = [r.copy() for r in kv]
    for r in kv2:
        r[Lt] = _bf16(np.full(r.shape[1], 3.0))
    alt = run(keys2, kv2)
    for a, b in zip(base, alt):
        for u in range(t + 1):
            assert np.array_equal(a["out"][u], b["out"][u]), (a["kind"], u)
        assert not np.array_equal(a["out"][t + 1], b["out"][t + 1]), a["kind"]


@pytest.mark.parametrize("shared", [False, True])
def test_every_position_selected_gives_dense_causal_attention(shared):
    """With P and k covering the whole context, token t attends to exactly
    the positions 0 .. L_t - 1 (its selection and its window, disjoint):
    textbook softmax(q V^T * scale) V over them (scipy)."""
    L, T, W = 150, 5, 20
    keys, idx_q, idx_w, attn_q, kv = _setup(6, L, T, D=64)
    res = oracle.decode_block("FU", keys, 0, L, T, W, L, L, idx_q, idx_w, attn_q,
                              lambda l, S: kv[l][S], 0.2, shared)
    for l, r in enumerate(res):
        V = oracle.fp4_dequantize(*oracle.fp4_quantize(kv[l]))
        for t, Lt in enumerate(oracle.block_lengths(L, T)):
            S = r["S"][t]
            assert len(set(S.tolist())) == len(S)
            if shared:
                # the block's selection is every position eligible for token 0;
                # token t adds its own window (the positions between are not
                # attended)
                E0 = L - T + 1 - W
                want = sorted(set(range(E0)) | set(range(Lt - W, Lt)))
            else:
                want = list(range(Lt))
            assert sorted(S.tolist()) == want
            rows = np.array(want)
            tt = 0.2 * (oracle.bf16_to_f64(attn_q[l][t]) @ V[rows].T)
            ref = scipy.special.softmax(tt, axis=1) @ V[rows]
            np.testing.assert_allclose(r["out"][t], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(r["lse"][t], scipy.special.logsumexp(tt, axis=1), rtol=0,
                                       atol=1e-12)
