"""Pins of the oracle's session functions (bounded replay bookkeeping): the
saved length drops exactly the newest min(R, L) positions, a saved state
restored elsewhere and completed by replaying the dropped tokens is the
original state, and a change inside the dropped window never reaches the
saved state while a change just before it does."""
import numpy as np
import pytest

import oracle


def _bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("L,R,want", [(1000, 128, 872), (128, 128, 0), (50, 128, 0), (0, 128, 0),
                                      (129, 128, 1), (7, 0, 7)])
def test_saved_length(L, R, want):
    assert oracle.session_saved_length(L, R) == want


def _state(seed, rows, n_layers=3, D=64):
    rng = np.random.default_rng(seed)
    x = [_bf16(rng.standard_normal((rows, D))) for _ in range(n_layers)]
    keys = rng.integers(-128, 128, size=(rows, 64)).astype(np.int8)
    fp4, sc = zip(*[oracle.fp4_quantize(xl) for xl in x])
    return x, keys, list(fp4), list(sc)


def test_restore_plus_replay_is_the_original_state():
    L, R, off = 700, 128, 40
    x, keys, fp4, sc = _state(1, off + L)
    saved = oracle.session_export(keys, fp4, sc, off, L, R)
    assert saved[0] == L - R
    # a fresh cache, the sequence now at another row offset
    new_off = 5
    keys2 = np.zeros((new_off + L + 10, 64), np.int8)
    fp42 = [np.zeros((new_off + L + 10, f.shape[1]), np.uint8) for f in fp4]
    sc2 = [np.zeros((new_off + L + 10, c.shape[1]), np.uint8) for c in sc]
    n = oracle.session_import(saved, keys2, fp42, sc2, new_off)
    assert n == L - R
    # replay: the dropped tokens' keys and latent rows, appended at n ..
    L2 = oracle.replay_append(keys2, fp42, sc2, new_off, n, keys[off + n:off + L],
                              [xl[off + n:off + L] for xl in x])
    assert L2 == L
    r_old, r_new = slice(off, off + L), slice(new_off, new_off + L)
    assert np.array_equal(keys2[r_new], keys[r_old])
    for a, b in zip(fp42 + sc2, fp4 + sc):
        assert np.array_equal(a[r_new], b[r_old])


def test_the_window_is_what_is_dropped():
    L, R = 300, 128
    x, keys, fp4, sc = _state(2, L)
    base = oracle.session_export(keys, fp4, sc, 0, L, R)
    k2, f2 = keys.copy(), [f.copy() for f in fp4]
    k2[L - R:] ^= 0x55                                   # the newest R positions
    f2[1][L - R:] ^= 0x0F
    alt = oracle.session_export(k2, f2, sc, 0, L, R)
    assert np.array_equal(base[1], alt[1]) and np.array_equal(base[2][1], alt[2][1])
    k3 = keys.copy()
    k3[L - R - 1] ^= 0x01                                # the last saved position
    assert not np.array_equal(oracle.session_export(k3, fp4, sc, 0, L, R)[1], base[1])


def test_short_sequences_keep_nothing():
    x, keys, fp4, sc = _state(3, 100)
    n, k, f, c = oracle.session_export(keys, fp4, sc, 0, 100, 128)
    assert n == 0 and k.shape == (0, 64) and all(a.shape[0] == 0 for a in f + c)
