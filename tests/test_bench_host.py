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
