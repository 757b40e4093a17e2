"""Pins of the oracle's sparse attention: dense softmax attention from scipy
when the selection covers the whole context, closed forms for a single row
and a zero query, order invariance, and the composed decode step."""
import math

import numpy as np
import pytest
import scipy.special

import oracle


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rand_rows(rng, n, D=512):
    x = _bf16(rng.standard_normal((n, D)))
    return oracle.fp4_quantize(x)


def test_dense_when_selection_covers_context():
    """k >= E: sparse attention over selection U window == textbook dense
    softmax(q V^T * scale) V over all L rows (scipy softmax / logsumexp)."""
    rng = np.random.default_rng(0)
    L, W, Hq, D = 300, 128, 8, 512
    codes, scales = _rand_rows(rng, L, D)
    q = _bf16(rng.standard_normal((Hq, D)))
    E = oracle.eligible_count(L, W)
    sel = np.arange(E)                       # every eligible position selected
    S = oracle.attention_positions(L, sel, W)
    assert sorted(S.tolist()) == list(range(L))
    out, lse = oracle.attention(q, codes[S], scales[S], 1 / math.sqrt(D))
    V = oracle.fp4_dequantize(codes, scales)
    t = (oracle.bf16_to_f64(q) @ V.T) / math.sqrt(D)
    ref = scipy.special.softmax(t, axis=1) @ V
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(t, axis=1), rtol=0, atol=1e-12)


def test_single_row_gives_the_row():
    rng = np.random.default_rng(1)
    codes, scales = _rand_rows(rng, 1)
    q = _bf16(rng.standard_normal((4, 512)))
    out, lse = oracle.attention(q, codes, scales, 0.1)
    v = oracle.fp4_dequantize(codes, scales)[0]
    assert np.array_equal(out, np.tile(v, (4, 1)))
    np.testing.assert_allclose(lse, 0.1 * (oracle.bf16_to_f64(q) @ v), rtol=1e-14)


def test_zero_query_gives_mean():
    rng = np.random.default_rng(2)
    codes, scales = _rand_rows(rng, 37)
    q = np.zeros((3, 512), dtype=np.uint16)
    out, lse = oracle.attention(q, codes, scales, 0.05)
    V = oracle.fp4_dequantize(codes, scales)
    np.testing.assert_allclose(out, np.tile(V.mean(axis=0), (3, 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(37), rtol=1e-14)


def test_order_invariance():
    rng = np.random.default_rng(3)
    codes, scales = _rand_rows(rng, 64)
    q = _bf16(rng.standard_normal((5, 512)))
    o1, l1 = oracle.attention(q, codes, scales, 1 / math.sqrt(512))
    perm = rng.permutation(64)
    o2, l2 = oracle.attention(q, codes[perm], scales[perm], 1 / math.sqrt(512))
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_two_rows_closed_form():
    """Two rows: out = (v0 + e^(t1 - t0) v1) / (1 + e^(t1 - t0))."""
    rng = np.random.default_rng(4)
    codes, scales = _rand_rows(rng, 2)
    q = _bf16(rng.standard_normal((1, 512)))
    out, lse = oracle.attention(q, codes, scales, 0.3)
    V = oracle.fp4_dequantize(codes, scales)
    qv = oracle.bf16_to_f64(q)[0]
    t0, t1 = 0.3 * (qv @ V[0]), 0.3 * (qv @ V[1])
    r = math.exp(t1 - t0)
    np.testing.assert_allclose(out[0], (V[0] + r * V[1]) / (1 + r), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], t0 + math.log1p(r), rtol=1e-13)


def test_empty_row_set():
    out, lse = oracle.attention(np.zeros((2, 512), np.uint16), np.zeros((0, 256), np.uint8),
                                np.zeros((0, 16), np.uint8), 0.1)
    assert not out.any() and np.isneginf(lse).all()


def test_decode_step_shared_kv():
    """One latent cache for every layer: two Reuse layers that attend with the
    same query see the same rows and give identical outputs, which layers with
    caches of their own do not."""
    rng = np.random.default_rng(6)
    L, W, P, k, H, Hq, D = 1200, 128, 200, 30, 4, 4, 512
    keys = rng.integers(-127, 128, size=(L, 64)).astype(np.int8)
    q0 = rng.integers(-127, 128, size=(H, 64)).astype(np.int8)
    w0 = rng.integers(0, 16, size=H).astype(np.int8)
    attn_q = [_bf16(rng.standard_normal((Hq, D))) for _ in range(4)]
    attn_q[3] = attn_q[2]
    kv0 = _bf16(rng.standard_normal((L, D)))
    kv_own = [_bf16(rng.standard_normal((L, D))) for _ in range(4)]
    args = ("FRUU", keys, 0, L, W, P, k, {0: q0, 1: q0}, {0: w0, 1: w0}, attn_q)
    shared = oracle.decode_step(*args, lambda l, S: kv0[S], 1 / math.sqrt(D))
    own = oracle.decode_step(*args, lambda l, S: kv_own[l][S], 1 / math.sqrt(D))
    assert np.array_equal(shared[2]["S"], shared[3]["S"])
    assert np.array_equal(shared[2]["out"], shared[3]["out"])
    assert np.array_equal(shared[2]["lse"], shared[3]["lse"])
    assert not np.allclose(own[2]["out"], own[3]["out"])


def test_decode_step_modes():
    """Full -> Reindex -> Reuse: a Reindex layer with the Full layer's own query
    selects the same positions; Reuse layers repeat the previous selection."""
    rng = np.random.default_rng(5)
    L, W, P, k, H, Hq, D = 1500, 128, 300, 40, 4, 4, 512
    keys = rng.integers(-127, 128, size=(L, 64)).astype(np.int8)
    q0 = rng.integers(-127, 128, size=(H, 64)).astype(np.int8)
    w0 = rng.integers(0, 16, size=H).astype(np.int8)
    q4 = rng.integers(-127, 128, size=(H, 64)).astype(np.int8)
    w4 = rng.integers(0, 16, size=H).astype(np.int8)
    idx_q = {0: q0, 1: q0, 4: q4}
    idx_w = {0: w0, 1: w0, 4: w4}
    attn_q = [_bf16(rng.standard_normal((Hq, D))) for _ in range(6)]
    kv_all = [_bf16(rng.standard_normal((L, D))) for _ in range(6)]
    res = oracle.decode_step("FRUURU", keys, 0, L, W, P, k, idx_q, idx_w, attn_q,
                             lambda l, S: kv_all[l][S], 1 / math.sqrt(D))
    assert [r["kind"] for r in res] == list("FRUURU")
    assert np.array_equal(res[0]["sel"], res[1]["sel"])
    assert np.array_equal(res[1]["sel"], res[2]["sel"]) and np.array_equal(res[2]["sel"], res[3]["sel"])
    # layer 4 re-scores layer 0's pool with its own query
    want = oracle.index_scores(keys, res[0]["pool_pos"], q4, w4)
    assert np.array_equal(res[4]["reindex_score"], want)
    assert np.array_equal(res[5]["sel"], res[4]["sel"])
    for r in res:
        assert len(r["S"]) == k + W
        assert len(set(r["S"].tolist())) == len(r["S"])
