"""Host-side checks of the benchmark's byte accounting: the algorithmic bytes
per step of each workload, from the call-by-call formulas (every buffer that
crosses the C ABI once, plus the index keys and FP4 rows the method reads)."""
import bench
from decode_kv_amd import workloads as W


def _mb(wl, lengths):
    ab = bench.algorithmic_bytes(wl, lengths)
    return {k: v / 1e6 for k, v in ab.items()}


def _close(got, want, tol=0.01):
    return all(abs(g - w) <= tol for g, w in zip(got, want))


def test_ctx_1m_bytes():
    wl = W.WORKLOADS["ctx_1m"]
    mb = _mb(wl, [1 << 20])
    # Full: 64 E + 65 H + 8 P;  E = 1,048,448
    assert bench.algorithmic_bytes(wl, [1 << 20])["scan_kernel"] == 64 * 1048448 + 65 * 64
    assert _close((mb["full"], mb["reindex"], mb["select"], mb["attn"], mb["append"]),
                  (67.24, 5.92, 0.80, 7.46, 0.0))
    assert _close([mb["step"]], [81.41])


def test_small_and_batched_bytes():
    assert _close([_mb(W.WORKLOADS["tiny_4k"], [4096])["step"]], [0.37])
    assert _close([_mb(W.WORKLOADS["single_64k"], [65536])["step"]], [4.83])
    mb = _mb(W.WORKLOADS["batch8_256k"], [262144] * 8)
    assert _close((mb["full"], mb["reindex"], mb["select"], mb["attn"], mb["step"]),
                  (135.23, 9.47, 2.13, 11.93, 158.80))
    # 4 layers x 8 sequences x (1,024 + 256 + 16) bytes, plus 8 index keys in and out
    assert bench.algorithmic_bytes(W.WORKLOADS["batch8_256k"], [262144] * 8)["append"] == \
        32 * 1296 + 8 * 128


def test_shared_kv_appends_one_row():
    per_layer = bench.algorithmic_bytes(W.WORKLOADS["ragged32_1m"], [5000])
    shared = bench.algorithmic_bytes(W.WORKLOADS["ragged32_1m_shared"], [5000])
    assert per_layer["append"] == 20 * 1296 + 128 and shared["append"] == 1296 + 128
    assert {k: v for k, v in per_layer.items() if k not in ("append", "step")} == \
        {k: v for k, v in shared.items() if k not in ("append", "step")}


def test_short_sequences_clamp():
    wl = W.WORKLOADS["ragged32_1m"]
    ab = bench.algorithmic_bytes(wl, [100])            # L <= W: no eligible position
    assert ab["full"] == 65 * wl.H and ab["reindex"] == 5 * 65 * wl.H
    assert ab["attn"] == 20 * (272 * 100 + 6 * 64 * 512)


def test_verify_block_bytes():
    """Five tokens at L = 2^20: the keys are read once (the last token's
    positions, or with a shared selection the first token's), each token
    brings its query, pool and selection, and the windows' union is 132 rows."""
    L, T, E4, E0 = 1 << 20, 5, (1 << 20) - 128, (1 << 20) - 132
    per = bench.algorithmic_bytes(W.WORKLOADS["ctx_1m_block5"], [L])
    sh = bench.algorithmic_bytes(W.WORKLOADS["ctx_1m_block5_shared"], [L])
    one = bench.algorithmic_bytes(W.WORKLOADS["ctx_1m"], [L])
    assert per["scan_kernel"] == 64 * E4 + T * 65 * 64
    assert sh["scan_kernel"] == 64 * E0 + T * 65 * 64
    assert per["full"] == 64 * E4 + T * 65 * 64 + T * 8 * 16384
    assert sh["full"] == 64 * E0 + T * 65 * 64 + 8 * 16384
    assert per["select"] == T * one["select"] and sh["select"] == one["select"]
    assert sh["attn"] == 20 * (272 * (512 + 132) + T * 6 * 64 * 512 + 4 * 512)
    # per-token selections counted once each, or by their union when given
    assert per["attn"] == 20 * (272 * (T * 512 + 132) + T * 6 * 64 * 512 + T * 4 * 512)
    uni = bench.algorithmic_bytes(W.WORKLOADS["ctx_1m_block5"], [L], [[600] * 20])
    assert uni["attn"] == 20 * (272 * (600 + 132) + T * 6 * 64 * 512 + T * 4 * 512)


def test_verify_block_appends_every_token():
    one = bench.algorithmic_bytes(W.WORKLOADS["batch8_256k"], [262144])
    blk = bench.algorithmic_bytes(W.WORKLOADS["batch8_256k_block5"], [262144])
    assert blk["append"] == 5 * one["append"]


def test_scan_bound_by_workload():
    """The scan's tightest bound at the peaks: one token streams 67 MB of keys
    (8.4 us at 8 TB/s) against 3.4 us of score-rule vector work; five tokens
    need 5 x 2 x 64 operations per position (17.1 us at 39.3 T lane-ops/s)
    and 256 prompt tokens 109 us, beyond their int8 matrix-core time."""
    peak = {"hbm": bench.HBM_PEAK_GBS * 1e9, "mfma": bench.INT8_PEAK_TOPS * 1e12,
            "alu": bench.ALU_PEAK_TOPS * 1e12}
    assert abs(bench.ALU_PEAK_TOPS - 39.3216) < 1e-9

    def times(name, lengths):
        ab = bench.algorithmic_bytes(W.WORKLOADS[name], lengths)
        return {"hbm": ab["scan_kernel"] / peak["hbm"], "mfma": ab["scan_ops"] / peak["mfma"],
                "alu": ab["scan_alu_ops"] / peak["alu"]}

    one = times("ctx_1m", [1 << 20])
    assert max(one, key=one.get) == "hbm" and abs(one["alu"] * 1e6 - 3.41) < 0.01
    blk = times("ctx_1m_block5", [1 << 20])
    assert max(blk, key=blk.get) == "alu" and abs(blk["alu"] * 1e6 - 17.07) < 0.01
    pf = times("prefill_128k_chunk256", [131072])
    assert max(pf, key=pf.get) == "alu" and 108 < pf["alu"] * 1e6 < 110
    # 64 int8 multiply-adds per head and position against 2 vector operations
    assert abs(pf["mfma"] / pf["alu"] - 64 * bench.ALU_PEAK_TOPS / bench.INT8_PEAK_TOPS) < 1e-9
