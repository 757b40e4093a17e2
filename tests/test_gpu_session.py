"""GPU parity of the multi-token append and of the session bookkeeping
(export, import, replay) against the oracle's session functions: every byte
of the saved and restored state must match, and a decode step after a
restore must give the same bits as one on the never-dropped caches."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_amd import csa2, pipeline
from decode_kv_amd import workloads as W
from test_gpu_parity import DEV, _say, u16

pytestmark = pytest.mark.gpu


def _bf16_rows(rng, shape):
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-8, 9, size=shape))).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("n,nl", [(7, 3), (50, 5)])
def test_append_tokens_matches_oracle(n, nl):
    """n tokens per sequence, nl layers, ragged start lengths: FP4 rows and
    index keys at len .. len + n - 1, len advanced by n, other rows untouched
    (21 rows per sequence take the one-workgroup kernel, 250 the wide one)."""
    rng = np.random.default_rng(n)
    B, D = 3, 512
    row_off = [0, 130, 260]
    lens = [0, 5, 70]
    rows = 400                                          # every appended row stays inside
    assert all(o + L + n <= nxt for o, L, nxt in zip(row_off, lens, row_off[1:] + [rows]))
    x = _bf16_rows(rng, (n, nl, B, D))
    kr = rng.integers(-128, 128, size=(n, B, 64)).astype(np.int8)
    fp4 = torch.full((nl, rows, D // 2), 0xA5, dtype=torch.uint8, device=DEV)
    sc = torch.full((nl, rows, D // 32), 0x5A, dtype=torch.uint8, device=DEV)
    keys = torch.full((rows, 64), 7, dtype=torch.int8, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    csa2.append_tokens(torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16),
                       torch.from_numpy(kr).to(DEV), torch.tensor(row_off, device=DEV), ln, fp4,
                       sc, keys)
    torch.cuda.synchronize()
    assert ln.cpu().tolist() == [L + n for L in lens]
    f, c, k = fp4.cpu().numpy(), sc.cpu().numpy(), keys.cpu().numpy()
    touched = np.zeros(rows, bool)
    for b in range(B):
        r = slice(row_off[b] + lens[b], row_off[b] + lens[b] + n)
        touched[r] = True
        assert np.array_equal(k[r], kr[:, b])
        for l in range(nl):
            codes, scales = oracle.fp4_quantize(x[:, l, b])
            assert np.array_equal(f[l, r], codes) and np.array_equal(c[l, r], scales), (b, l)
    assert (k[~touched] == 7).all() and (f[:, ~touched] == 0xA5).all() and (c[:, ~touched] == 0x5A).all()


def _random_caches(rng, rows, nl, D=512):
    keys = rng.integers(-128, 128, size=(rows, 64)).astype(np.int8)
    fp4 = rng.integers(0, 256, size=(nl, rows, D // 2)).astype(np.uint8)
    sc = rng.integers(0, 255, size=(nl, rows, D // 32)).astype(np.uint8)
    return keys, fp4, sc


@pytest.mark.parametrize("pinned,nl", [(False, 4), (True, 4), (False, 1)])
def test_session_export_import(pinned, nl):
    """Ragged lengths (0, shorter than the window, window + 1, long), saved to
    device or pinned host memory, restored at other row offsets; four layers'
    caches, or the one cache of the shared-KV layout."""
    rng = np.random.default_rng(2 + nl)
    R = 128
    lens = [0, 50, 128, 129, 5000]
    B = len(lens)
    row_off = list(np.cumsum([0] + [L + 3 for L in lens[:-1]]))
    rows = row_off[-1] + lens[-1] + 3
    keys, fp4, sc = _random_caches(rng, rows, nl)
    cap = max(oracle.session_saved_length(L, R) for L in lens)
    kw = dict(device="cpu", pin_memory=True) if pinned else dict(device=DEV)
    s_keys = torch.full((B, cap, 64), -3, dtype=torch.int8, **kw)
    s_fp4 = torch.full((nl, B, cap, 256), 0xEE, dtype=torch.uint8, **kw)
    s_sc = torch.full((nl, B, cap, 16), 0xEE, dtype=torch.uint8, **kw)
    s_len = torch.full((B,), -1, dtype=torch.int32, **kw)
    d = lambda a: torch.from_numpy(a).to(DEV)
    ro = torch.tensor(row_off, dtype=torch.int64, device=DEV)
    csa2.session_export(ro, torch.tensor(lens, dtype=torch.int32, device=DEV), R, d(fp4), d(sc),
                        d(keys), s_fp4, s_sc, s_keys, s_len)
    torch.cuda.synchronize()
    got_k, got_f, got_s = s_keys.cpu().numpy(), s_fp4.cpu().numpy(), s_sc.cpu().numpy()
    assert s_len.cpu().tolist() == [oracle.session_saved_length(L, R) for L in lens]
    for b, L in enumerate(lens):
        n, k, f, c = oracle.session_export(keys, list(fp4), list(sc), row_off[b], L, R)
        assert np.array_equal(got_k[b, :n], k) and (got_k[b, n:] == -3).all(), b
        for l in range(nl):
            assert np.array_equal(got_f[l, b, :n], f[l]) and (got_f[l, b, n:] == 0xEE).all()
            assert np.array_equal(got_s[l, b, :n], c[l]) and (got_s[l, b, n:] == 0xEE).all()
    # restore at other offsets into fresh caches
    new_off = list(np.cumsum([17] + [L + 11 for L in lens[:-1]]))
    rows2 = new_off[-1] + lens[-1] + 11
    k2 = torch.full((rows2, 64), 9, dtype=torch.int8, device=DEV)
    f2 = torch.full((nl, rows2, 256), 0x11, dtype=torch.uint8, device=DEV)
    c2 = torch.full((nl, rows2, 16), 0x22, dtype=torch.uint8, device=DEV)
    ln2 = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    csa2.session_import(torch.tensor(new_off, dtype=torch.int64, device=DEV), ln2, s_len, s_fp4,
                        s_sc, s_keys, f2, c2, k2)
    torch.cuda.synchronize()
    assert ln2.cpu().tolist() == s_len.cpu().tolist()
    k2n, f2n, c2n = k2.cpu().numpy(), f2.cpu().numpy(), c2.cpu().numpy()
    ref_k = np.full_like(k2n, 9)
    ref_f = np.full_like(f2n, 0x11)
    ref_c = np.full_like(c2n, 0x22)
    for b, L in enumerate(lens):
        saved = oracle.session_export(keys, list(fp4), list(sc), row_off[b], L, R)
        oracle.session_import(saved, ref_k, list(ref_f), list(ref_c), new_off[b])
    assert np.array_equal(k2n, ref_k) and np.array_equal(f2n, ref_f) and np.array_equal(c2n, ref_c)


def test_session_resume_decode_step():
    """An appending workload runs two steps; its sessions are saved, restored
    into a second engine's zeroed caches, and the dropped windows replayed
    with csa2_append_tokens from the generator's rows (what the model would
    recompute).  The restored caches equal the originals byte for byte, and
    the next decode step gives identical bits on both engines."""
    wl = W.WORKLOADS["ragged32_1m"].scaled(B=4, len_range=(300, 30000), n_layers=5, steps=3)
    R = wl.window
    case = W.Case(wl, 4, DEV)
    a = pipeline.Engine(case, DEV)
    for step in range(2):
        a.run_step(a.step_inputs(step))
    torch.cuda.synchronize()
    lens = a.lens.cpu().tolist()
    cap = max(oracle.session_saved_length(L, R) for L in lens)
    nl = wl.n_kv
    s_keys = torch.empty((wl.B, cap, 64), dtype=torch.int8, device=DEV)
    s_fp4 = torch.empty((nl, wl.B, cap, 256), dtype=torch.uint8, device=DEV)
    s_sc = torch.empty((nl, wl.B, cap, 16), dtype=torch.uint8, device=DEV)
    s_len = torch.empty((wl.B,), dtype=torch.int32, device=DEV)
    csa2.session_export(a.row_off, a.lens, R, a.kv_fp4, a.kv_scale, a.keys, s_fp4, s_sc, s_keys,
                        s_len)
    b_eng = pipeline.Engine(W.Case(wl, 4, DEV), DEV)
    b_eng.kv_fp4.zero_()
    b_eng.kv_scale.zero_()
    b_eng.keys.zero_()
    b_eng.lens.fill_(-1)
    csa2.session_import(b_eng.row_off, b_eng.lens, s_len, s_fp4, s_sc, s_keys, b_eng.kv_fp4,
                        b_eng.kv_scale, b_eng.keys)
    torch.cuda.synchronize()
    assert b_eng.lens.cpu().tolist() == [L - R for L in lens]
    for b, L in enumerate(lens):                        # replay the dropped window
        pos = list(range(L - R, L))
        x = torch.stack([case.kv_bf16(l, b, pos) for l in range(nl)]).transpose(0, 1)
        x = x.reshape(R, nl, 1, wl.D).contiguous()
        off = int(a.row_off[b])
        kr = a.keys[off + L - R:off + L].reshape(R, 1, 64).contiguous()
        csa2.append_tokens(x, kr, b_eng.row_off[b:b + 1], b_eng.lens[b:b + 1], b_eng.kv_fp4,
                           b_eng.kv_scale, b_eng.keys)
    torch.cuda.synchronize()
    assert b_eng.lens.cpu().tolist() == lens
    for b, L in enumerate(lens):
        off = int(a.row_off[b])
        r = slice(off, off + L)
        assert torch.equal(a.keys[r], b_eng.keys[r]), b
        assert torch.equal(a.kv_fp4[:, r], b_eng.kv_fp4[:, r]), b
        assert torch.equal(a.kv_scale[:, r], b_eng.kv_scale[:, r]), b
    inp = a.step_inputs(2)
    a.run_step(inp)
    b_eng.run_step(inp)
    torch.cuda.synchronize()
    for n in ("pool_pos", "pool_score", "sel_pos", "sel_len", "out", "lse", "lens"):
        assert torch.equal(getattr(a, n), getattr(b_eng, n)), n
    _say("  resumed", wl.B, "sessions, lengths", lens)
