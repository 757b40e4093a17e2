"""The seeded generator: torch implementation equals the plain-integer
SplitMix64 definition, streams are reproducible, and the workloads have the
stated shapes and structure."""
import math

import numpy as np
import torch

from decode_kv_amd import inputs as I
from decode_kv_amd import workloads as W


def test_splitmix64_known_value():
    # SplitMix64 seeded with 0: the first output is 0xE220A8397B1DCDAF
    assert I.splitmix64_py(0) == 0xE220A8397B1DCDAF


def test_torch_hash_matches_plain_integers():
    key = I.stream_key(123, 4, 5)
    idx = torch.tensor([0, 1, 2, 1000, 2 ** 40 + 7, 2 ** 62], dtype=torch.int64)
    got = I.hash_stream(key, idx).tolist()
    for i, g in zip(idx.tolist(), got):
        want = I.splitmix64_py((key + i * I.GOLDEN) & I.MASK64)
        assert (g & I.MASK64) == want


def test_streams_reproducible_and_distinct():
    a = I.bf16_normal(I.stream_key(1, 2), 0, 4096, "cpu")
    b = I.bf16_normal(I.stream_key(1, 2), 0, 4096, "cpu")
    c = I.bf16_normal(I.stream_key(1, 3), 0, 4096, "cpu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    sub = I.bf16_normal(I.stream_key(1, 2), 1000, 100, "cpu")
    assert torch.equal(sub.view(torch.int16), a[1000:1100].view(torch.int16))
    f = a.float()
    assert abs(f.mean().item()) < 0.1 and abs(f.std().item() - 1) < 0.1


def test_int8_distributions():
    u = I.int8_uniform(I.stream_key(0, 9), 0, 100000, "cpu")
    assert u.min().item() == -127 and u.max().item() == 127
    g = I.int8_normal(I.stream_key(0, 10), 0, 100000, 30.0, "cpu").float()
    assert abs(g.std().item() - 30) < 1.5


def test_workload_shapes():
    wl = W.WORKLOADS["ctx_1m"]
    assert wl.pattern == "FRUURUUURUUURUUURUUU"
    assert W.WORKLOADS["batch8_256k"].pattern == "FRUU"
    c = W.Case(W.WORKLOADS["ragged32_1m"], seed=0)
    assert len(c.lengths) == 32
    assert all(4096 <= L <= 1048576 for L in c.lengths)
    assert c.caps[0] == c.lengths[0] + 64
    assert c.row_off[1] == c.caps[0]


def test_case_planted_and_kv_rows():
    wl = W.WORKLOADS["tiny_4k"]
    c = W.Case(wl, seed=3)
    keys = c.keys_seq(0)
    pos, rows = c.planted(0)
    assert len(pos) == 8 and len(set(pos.tolist())) == 8
    assert pos.max() < 4096 - 128
    assert torch.equal(keys[torch.as_tensor(pos)], torch.as_tensor(rows))
    kv = c.kv_bf16(0, 0, [5, 17])
    ids = c.kv_row_id(0, 0, [5, 17])
    assert ids.min() >= 0 and ids.max() < W.KV_POOL_ROWS
    pr = c.kv_pool_range(int(ids[0]), 1)
    assert torch.equal(kv[0].view(torch.int16), pr[0].view(torch.int16))
    assert not torch.equal(c.kv_bf16(1, 0, [5]).view(torch.int16), kv[:1].view(torch.int16))


def test_log_distance_planting():
    wl = W.WORKLOADS["ctx_1m"].scaled(L=50000)
    c = W.Case(wl, seed=1)
    pos, rows = c.planted(0)
    assert len(pos) == 1024 and len(set(pos.tolist())) == 1024
    d = 50000 - pos
    assert d.min() >= 129
    # log-uniform distances: roughly equal counts per decade
    assert (d < 1000).sum() > 200 and (d > 10000).sum() > 200


def test_planted_positions_of_short_sequences():
    """Sequences with fewer eligible positions than planted keys plant every
    eligible position (the log-distance draw cannot reach position 0), and
    one more eligible position than planted keys still finishes."""
    wl = W.WORKLOADS["ragged32_1m"].scaled(B=2, len_range=(200, 400), n_layers=1)
    c = W.Case(wl, 3, "cpu")
    for b in range(wl.B):
        E = max(0, c.lengths[b] - wl.window)
        pos, rows = c.planted(b)
        assert sorted(pos.tolist()) == list(range(min(E, wl.n_planted)))
        assert rows.shape == (len(pos), wl.Dk)
    wl2 = W.WORKLOADS["ctx_1m"].scaled(L=wl.n_planted + 1 + wl.window, n_planted=wl.n_planted)
    pos, _ = W.Case(wl2, 0, "cpu").planted(0)
    assert len(set(pos.tolist())) == wl.n_planted and pos.max() <= wl.n_planted
