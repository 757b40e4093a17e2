"""Decode-step benchmark of the CSA2 sparse-attention path on one MI355X.

Workload (default): ctx_1m -- one sequence at L = 1,048,576 cached tokens,
20 decoder layers F R U U R U U U R ... (Full once, Reindex at layer 1 and
every 4th layer, Reuse otherwise), pool P = 16,384, top-k 512, window 128,
64 int8 index heads x 64, 64 bf16 query heads x 512, FP4 E2M1 latent KV with
E8M0 scales per 32 elements.  Synthetic seeded inputs.  --workload picks any
workload of decode_kv_amd/workloads.py (tiny_4k, single_64k, batch8_256k,
ctx_1m, ragged32_1m, their *_shared variants, verify blocks *_block5 and
*_block5_shared, prefill_128k_chunk256).

A step is the whole hot path: for workloads with appends, the new token of
every sequence is written into every layer's FP4 cache and the index-key
cache first (csa2_append_token); then the Full index scan + pool, the top-k
selections, the Reindex passes and every layer's sparse attention.  The step
is captured once in a HIP graph and replayed.  Appending workloads replay it
over consecutive decode steps: the lengths advance on the device, and each
step's inputs (re-drawn queries, the new token's rows) are copied into the
graph's input buffers before the step, outside the timed region.

Cold timing (the headline) evicts the 256 MB Infinity Cache before every
step with an untimed read of a 1 GiB buffer; warm timing (reported beside it)
does not.  Each step is timed with HIP events on the replay stream.

The roofline object covers the Full scan's scoring kernel, the one kernel of
the step that streams the whole context (64 B of index key per position),
against the tightest of three bounds at the peaks: its key bytes at HBM
speed, its int8 multiply-adds at the matrix-core rate and its score-rule
vector operations (a max and a multiply-add per token, position and head) at
the integer ALU rate; the other two are listed beside it.  One token is
HBM-bound; a block of query tokens is ALU-bound.  The kernel's average
launch duration comes from back-to-back launches through
csa2_index_score, captured in one HIP graph, each over a key copy that is not
in the Infinity Cache.  read_ceiling is the same measurement for a kernel that
only reads the key bytes (csa2_stream_read) in the scoring kernel's launch
shape.  attention_roofline prices each layer's attention call (the attention
kernel and its combine) the same way, from cold calls timed one by one: the
step spends most of its time there, far below HBM speed, because at these
sizes the call is bound by launch and memory latency, not by bytes.
per_call_us times one eager step call by call.

Output: one JSON line (metric, value = steps/s, roofline, CPU-oracle
baseline, ...).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0          # dense int8 MFMA, MI355X
# integer vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one operation per
# lane-instruction (the fp32 vector peak, 157.3 TFLOP/s, counts a packed FMA
# as four flops per lane-instruction)
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "decode steps/s at 1M ctx (index+sparse attn) + achieved HBM GB/s vs peak"


def algorithmic_bytes(wl, lengths, sel_union=None) -> dict:
    """Bytes the method must move per step (every buffer crossing the C ABI
    once, plus the index keys and KV rows it reads), summed over sequences.

    A verify block of T tokens reads the index keys once for all tokens (the
    positions the last token may rank, or with a shared selection those of the
    first token) and the union of the tokens' windows (window + T - 1 rows).
    sel_union[b][l], when given, is the number of distinct positions in the T
    per-token selections layer l attends with; without it each token's
    selection is counted on its own."""
    pat = wl.pattern
    nF, nR = pat.count("F"), pat.count("R")
    T, shared = wl.block, wl.block_shared or wl.block == 1
    tot = {"append": 0, "full": 0, "select": 0, "reindex": 0, "attn": 0, "scan_kernel": 0}
    for b, L in enumerate(lengths):
        Ls = [L - (T - 1 - t) for t in range(T)]
        Es = [max(0, x - wl.window) for x in Ls]
        E_scan = Es[0] if shared else Es[-1]
        lists = [Es[0]] if shared else Es                      # eligible count of each list
        peff = [min(wl.P, e) for e in lists]
        keff = [min(wl.k, p) for p in peff]
        q_idx = T * 65 * wl.H                                  # int8 query + weights per token
        tot["full"] += nF * (64 * E_scan + q_idx + 8 * sum(peff))
        tot["select"] += (nF + nR) * sum(8 * p + 4 * kk for p, kk in zip(peff, keff))
        tot["reindex"] += nR * (72 * sum(peff) + q_idx)
        win_rows = min(wl.window + T - 1, max(0, L))
        for l in range(wl.n_layers):
            if shared:
                sel_rows = keff[0]
            elif sel_union is not None:
                sel_rows = sel_union[b][l]
            else:
                sel_rows = sum(keff)
            tot["attn"] += 272 * (sel_rows + win_rows) + T * 6 * wl.Hq * wl.D + 4 * sum(keff)
        tot["scan_kernel"] += 64 * E_scan + q_idx
        # int8 multiply-adds of the scan (two operations each): every token of
        # the block against the positions it ranks
        scan_E = Es[0] * T if shared else sum(Es)
        tot["scan_ops"] = tot.get("scan_ops", 0) + 2 * wl.Dk * wl.H * scan_E
        # and the vector work of the score rule per token, position and head:
        # the ReLU (a max) and the weighted accumulate (a multiply-add)
        tot["scan_alu_ops"] = tot.get("scan_alu_ops", 0) + 2 * wl.H * scan_E
        if wl.append:
            # per token and cache (one per layer, or one shared by all): the
            # bf16 row in, its FP4 codes and scales out; the 64-byte index key
            # in and out
            tot["append"] += T * (wl.n_kv * (2 * wl.D + wl.D // 2 + wl.D // 32) + 2 * wl.Dk)
    tot.setdefault("scan_ops", 0)
    tot.setdefault("scan_alu_ops", 0)
    tot["step"] = tot["append"] + tot["full"] + tot["select"] + tot["reindex"] + tot["attn"]
    return tot


def selection_unions(eng) -> list:
    """Per sequence and layer: distinct positions in the block's per-token
    selections that the layer attends with (from the engine's last step)."""
    import numpy as np
    wl = eng.wl
    T = wl.block
    sel = eng.sel_pos.cpu().numpy()
    sl = eng.sel_len.cpu().numpy()
    out = []
    for b in range(wl.B):
        row = []
        for l in range(wl.n_layers):
            src = eng.selection_layer(l)
            parts = [sel[src, b * T + t, :sl[src, b * T + t]] for t in range(T)]
            row.append(len(np.unique(np.concatenate(parts))) if parts else 0)
        out.append(row)
    return out


SCAN_SOURCES = ("decode_kv_amd/csrc/index_full.hip", "decode_kv_amd/csrc/common.h")


def scan_source_hash() -> str:
    """sha256 over the scanning kernel's sources (the file that holds it and
    the shared device helpers it uses)."""
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def stale_traffic(profile_path: str):
    """HBM traffic of the scan kernel from a committed counter summary, or
    None if the kernel's sources changed since the counters were taken."""
    try:
        rec = json.load(open(profile_path))
        if rec.get("source_sha256") != scan_source_hash():
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


def attention_roofline(ab: dict, wl, call_us: float, calls: int) -> dict:
    """The attention call (sparse_attn_kernel and attn_combine_kernel) of one
    layer against HBM: its algorithmic bytes (selected and window FP4 rows,
    queries, selection entries and fp32 outputs) over its measured cold call
    time.  Its bf16 products need far less time at the matrix-core peak than
    its bytes at the HBM peak, so HBM is the bound it is priced against."""
    per_call = ab["attn"] / wl.n_layers
    gbs = per_call / (call_us * 1e-6) / 1e9
    return {"kernel": "sparse_attn_kernel + attn_combine_kernel (one attention call per layer, "
                      "Infinity Cache evicted before each)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 5), "avg_call_us": round(call_us, 3),
            "calls_timed": calls, "algorithmic_bytes_per_call": round(per_call)}


def cpu_baseline(wl, seed: int, step: int, keys_np, seconds_target: float = 12.0) -> dict:
    """The oracle, untuned, timed on the host cores on decode steps of the
    same workload.  One sequence: whole steps repeated while under the time
    target (median).  A batch: the sequences of one step in order until the
    time target, the step's time extrapolated by the share of cached
    positions they hold (the Full scan, linear in the length, dominates)."""
    import numpy as np
    import torch

    import oracle
    from decode_kv_amd import workloads as W
    oracle.build(force=False)
    case = W.Case(wl, seed, "cpu")
    lens = case.lengths_at(step)
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    T = wl.block
    FR = [l for l, c in enumerate(wl.pattern) if c in "FR"]

    def per_token(fn, conv, l, b):
        if T == 1:
            return conv(fn(step, l, b))
        return np.stack([conv(fn(step, l, b, t)) for t in range(T)])

    def seq_inputs(b):
        idx_q = {l: per_token(case.index_q, lambda x: x.numpy(), l, b) for l in FR}
        idx_w = {l: per_token(case.index_w, lambda x: x.numpy(), l, b) for l in FR}
        attn_q = [per_token(case.attn_q, u16, l, b) for l in range(wl.n_layers)]
        off = int(case.row_off[b])
        return keys_np[off:off + case.caps[b]], idx_q, idx_w, attn_q, \
            (lambda l, S, b=b: u16(case.kv_bf16(l, b, S)))

    # a long block with per-token selection (a prefill chunk): the oracle runs
    # its last Ts tokens, whose work per token is the same as the others', and
    # the time is scaled by T / Ts
    Ts = 8 if (T > 16 and not wl.block_shared) else T

    def run(b, inputs):
        kb, idx_q, idx_w, attn_q, kv_rows = inputs
        t0 = time.perf_counter()
        if T == 1:
            oracle.decode_step(wl.pattern, kb, 0, lens[b], wl.window, wl.P, wl.k, idx_q, idx_w,
                               attn_q, kv_rows, wl.sm_scale)
        else:
            sub = lambda d: {l: v[T - Ts:] for l, v in d.items()}
            oracle.decode_block(wl.pattern, kb, 0, lens[b], Ts, wl.window, wl.P, wl.k,
                                sub(idx_q), sub(idx_w), [a[T - Ts:] for a in attn_q], kv_rows,
                                wl.sm_scale, wl.block_shared)
        return (time.perf_counter() - t0) * T / Ts

    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    t_all = time.perf_counter()
    if wl.B == 1:
        inputs = seq_inputs(0)
        times = []
        while True:
            times.append(run(0, inputs))
            if time.perf_counter() - t_all + times[-1] > seconds_target or len(times) >= 50:
                break
        per = statistics.median(times)
        sample = ("%d full decode step(s) of the same workload (1 sequence, L=%d, %d layers), "
                  "median %.2f s/step" % (len(times), lens[0], wl.n_layers, per))
        if Ts < T:
            sample = ("%d run(s) of the last %d of the block's %d tokens (1 sequence, L=%d, %d "
                      "layers), scaled by %d/%d: median %.2f s per step"
                      % (len(times), Ts, T, lens[0], wl.n_layers, T, Ts, per))
    else:
        t_done, L_done, n_done = 0.0, 0, 0
        for b in range(wl.B):
            t_done += run(b, seq_inputs(b))
            L_done += lens[b]
            n_done += 1
            if time.perf_counter() - t_all > seconds_target:
                break
        per = t_done * sum(lens) / max(1, L_done)
        sample = ("%d of %d sequences of decode step %d (%d of %d cached positions, %d layers) "
                  "in %.2f s; step time scaled by the share of positions: %.2f s/step"
                  % (n_done, wl.B, step, L_done, sum(lens), wl.n_layers, t_done, per))
    return {"value": round(1.0 / per, 5), "unit": "decode steps/s", "cores": cores,
            "kind": "oracle", "sample": sample}


def session_measure(eng, case, stream, reps: int = 10) -> dict:
    """Bounded-replay bookkeeping on the engine's caches: save every
    sequence's state (all but the newest `window` positions), restore it in
    place, and replay the dropped window with one multi-token append (the
    rows the model would recompute come from the generator).  HIP events
    around each call on `stream`; the caches end as they began."""
    import torch

    from decode_kv_amd import csa2
    wl = eng.wl
    R = wl.window
    dev = eng.keys.device
    lens = eng.lens.cpu().tolist()
    if min(lens) < R:
        return {"skipped": "a sequence is shorter than the replay window"}
    saved = [L - R for L in lens]
    cap, nl = max(saved), wl.n_kv
    s_keys = torch.empty((wl.B, cap, wl.Dk), dtype=torch.int8, device=dev)
    s_fp4 = torch.empty((nl, wl.B, cap, wl.D // 2), dtype=torch.uint8, device=dev)
    s_sc = torch.empty((nl, wl.B, cap, wl.D // 32), dtype=torch.uint8, device=dev)
    s_len = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    # replay inputs: token j of sequence b is position L_b - R + j
    x = torch.stack([torch.stack([case.kv_bf16(l, b, list(range(L - R, L)))
                                  for b, L in enumerate(lens)]) for l in range(nl)])
    x = x.permute(2, 0, 1, 3).contiguous()                       # [R][n_kv][B][D]
    kr = torch.stack([eng.keys[int(eng.row_off[b]) + L - R:int(eng.row_off[b]) + L]
                      for b, L in enumerate(lens)]).transpose(0, 1).contiguous()
    keys0 = eng.keys.clone()
    fp40, sc0 = eng.kv_fp4.clone(), eng.kv_scale.clone()
    t = {"export": [], "import": [], "replay": []}
    for _ in range(reps):
        with torch.cuda.stream(stream):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            csa2.session_export(eng.row_off, eng.lens, R, eng.kv_fp4, eng.kv_scale, eng.keys,
                                s_fp4, s_sc, s_keys, s_len, stream)
            ev[1].record()
            csa2.session_import(eng.row_off, eng.lens, s_len, s_fp4, s_sc, s_keys, eng.kv_fp4,
                                eng.kv_scale, eng.keys, stream)
            ev[2].record()
            csa2.append_tokens(x, kr, eng.row_off, eng.lens, eng.kv_fp4, eng.kv_scale, eng.keys,
                               stream)
            ev[3].record()
        torch.cuda.synchronize()
        for i, k in enumerate(("export", "import", "replay")):
            t[k].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    assert eng.lens.cpu().tolist() == lens, "replay did not restore the lengths"
    assert torch.equal(eng.keys, keys0) and torch.equal(eng.kv_fp4, fp40) and \
        torch.equal(eng.kv_scale, sc0), "save, restore and replay changed the caches"
    row = wl.Dk + nl * (wl.D // 2 + wl.D // 32)                # bytes per saved position
    moved = 2 * sum(saved) * row                               # read once, written once
    replay_bytes = wl.B * R * (nl * (2 * wl.D + wl.D // 2 + wl.D // 32) + 2 * wl.Dk)
    med = {k: statistics.median(v) for k, v in t.items()}
    return {
        "replay_window": R, "saved_positions": sum(saved), "bytes_per_position": row,
        "saved_MB": round(sum(saved) * row / 1e6, 1),
        "dropped_MB": round(wl.B * R * row / 1e6, 3),
        "export_us": round(med["export"], 1), "import_us": round(med["import"], 1),
        "replay_append_us": round(med["replay"], 1),
        "export_GBps": round(moved / (med["export"] * 1e-6) / 1e9, 1),
        "import_GBps": round(moved / (med["import"] * 1e-6) / 1e9, 1),
        "replay_GBps": round(replay_bytes / (med["replay"] * 1e-6) / 1e9, 1),
        "note": "device-to-device copies (HBM read + write counted); replay appends the "
                "dropped window's rows in one csa2_append_tokens call; median of %d" % reps,
    }


def measure_overheads() -> dict:
    """The cost of a dependent kernel node in a captured graph (a chain of
    empty kernels) and of handing split partials to a merge in a second kernel
    versus inside one kernel (csa2_handoff), at the attention's one-sequence
    shape (4 head groups x 20 splits) and a wider one (8 x 16)."""
    import torch

    from decode_kv_amd import csa2
    stream = torch.cuda.Stream()

    def graph_us(fn, n, reps=5):
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        best = None
        for _ in range(reps):
            with torch.cuda.stream(stream):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e3 / n
            best = t if best is None else min(best, t)
        return best

    res = {}
    for n in (55, 110):
        res["graph_node_us_%d_nodes" % n] = round(
            graph_us(lambda: [csa2.empty_kernel(stream) for _ in range(n)], n), 3)
    ho = {}
    for groups, splits in ((4, 20), (8, 16)):
        scratch = torch.zeros(csa2.handoff_scratch_bytes(groups, splits), dtype=torch.uint8,
                              device="cuda")
        out = torch.zeros((groups, 8192), dtype=torch.float32, device="cuda")
        ref = None
        row = {}
        for mode, name in ((0, "two_kernels"), (1, "one_kernel_write_through_counter"),
                           (2, "one_kernel_device_fences")):
            iters = 50
            us = graph_us(lambda: [csa2.handoff(mode, groups, splits, 1.0 + (i % 7), scratch, out,
                                                stream) for i in range(iters)], iters)
            got = out.clone()
            ok = bool(torch.isfinite(got).all())
            if ref is None:
                ref = got
            row[name] = {"us_per_handoff": round(us, 3), "finite": ok,
                         "same_as_two_kernels": bool(torch.equal(got, ref))}
        ho["%d_groups_x_%d_splits" % (groups, splits)] = row
    res["handoff"] = ho
    res["note"] = ("graph of dependent empty kernels (per node), and 50 hand-offs of 32 KiB "
                   "partials per workgroup captured in one graph (per hand-off); best of 5 "
                   "replays, HIP events on the replay stream")
    return res


def say(msg: str):
    """Progress line on stderr (the JSON result is the only stdout line)."""
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps per mode (default 50; 64 for appending workloads)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ctx_1m")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-only", action="store_true", help="skip the warm-mode timing")
    ap.add_argument("--no-session", action="store_true",
                    help="skip the session save / restore / replay measurement")
    ap.add_argument("--overheads", action="store_true",
                    help="only measure the kernel-node and partial hand-off costs (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_kv_amd import csa2, pipeline
    from decode_kv_amd import workloads as W

    assert torch.cuda.is_available(), "no GPU"
    csa2.lib()
    if args.overheads:
        print(json.dumps({"overheads": measure_overheads()}), flush=True)
        return
    dev = torch.device("cuda:0")
    wl0 = W.WORKLOADS[args.workload]
    K = args.steps if args.steps is not None else (64 if wl0.append else 50)
    Wm = args.warmup
    modes = ["cold"] + ([] if args.cold_only else ["warm"])
    n_eager = 2
    # appending workloads reserve one position per executed step: eager
    # warm-up, the call-by-call pass, and warm-up + timed steps of each mode
    wl = wl0.scaled(steps=n_eager + 1 + len(modes) * (Wm + K)) if wl0.append else wl0
    t_setup = time.perf_counter()
    case = W.Case(wl, args.seed, dev)
    eng = pipeline.Engine(case, dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        static = eng.step_inputs(0)
    torch.cuda.synchronize()
    say("setup %.1f s" % (time.perf_counter() - t_setup))

    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scrub_sink = torch.empty((), dtype=torch.int64, device=dev)

    def evict():
        torch.sum(scrub.view(torch.int64), dim=0, out=scrub_sink)

    next_step = [0]

    def prepare():
        """Make the static inputs those of the next decode step (appending
        workloads; on the current stream, before any timing event)."""
        i = next_step[0]
        next_step[0] += 1
        if wl.append and i > 0:
            pipeline.copy_inputs(static, eng.step_inputs(i))
        return i

    # eager warm-up
    with torch.cuda.stream(stream):
        for _ in range(n_eager):
            prepare()
            eng.run_step(static)
    torch.cuda.synchronize()
    ref_out = eng.out.clone()

    # ---- the scoring kernel alone (csa2_index_score: the Full scan's key
    # streaming stage) and a plain read of the same keys (csa2_stream_read):
    # n_scan launches captured back to back in one HIP graph (so no host
    # launch gap is timed), one event pair around the replay on the replay
    # stream.  Launch i reads key copy i mod R; R copies exceed the 256 MB
    # Infinity Cache, so every launch streams its keys from HBM.
    key_bytes = eng.keys.numel() * eng.keys.element_size()
    R = max(2, -(-(300 << 20) // key_bytes) + 1)
    key_copies = [eng.keys] + [eng.keys.clone() for _ in range(R - 1)]
    q0, w0 = static["idx_q"][0], static["idx_w"][0]
    blk = wl.block > 1
    n_lists = wl.B if (not blk or wl.block_shared) else wl.B * wl.block
    scores = torch.empty((n_lists, eng.max_len), dtype=torch.int32, device=dev)
    sink = torch.empty(csa2.stream_read_sink_words(key_bytes), dtype=torch.int32, device=dev)
    n_scan = max(50, 4 * R)

    def scan_all():
        for i in range(n_scan):
            if blk:
                csa2.index_score_block(q0, w0, key_copies[i % R], eng.row_off, eng.lens,
                                       eng.max_len, eng.total_len, wl.window, wl.block_shared,
                                       scores, eng.ws_full, stream)
            else:
                csa2.index_score(q0, w0, key_copies[i % R], eng.row_off, eng.lens, eng.max_len,
                                 eng.total_len, wl.window, scores, eng.ws_full, stream)

    def read_all():
        for i in range(n_scan):
            csa2.stream_read(key_copies[i % R], sink, stream)

    def graph_avg_ms(fn):
        with torch.cuda.stream(stream):
            fn()                                    # eager warm-up
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        with torch.cuda.stream(stream):
            g.replay()
            evict()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            g.replay()
            s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / n_scan

    scan_avg_ms = graph_avg_ms(scan_all)
    read_avg_ms = graph_avg_ms(read_all)
    del key_copies, scores
    say("scan kernel %.2f us, plain read %.2f us per launch" % (scan_avg_ms * 1e3, read_avg_ms * 1e3))

    # ---- one eager step, call by call: the GPU is first held busy long enough
    # for the host to queue the whole step, so the events between the calls
    # measure GPU time only
    per_call = {}
    with torch.cuda.stream(stream):
        prepare()
        evict()
        torch.cuda._sleep(50_000_000)
        e_prev = torch.cuda.Event(enable_timing=True)
        e_prev.record()
        marks = []

        def mark(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append((name, e))

        eng.run_step(static, mark=mark)
    torch.cuda.synchronize()
    for name, e in marks:
        rec = per_call.setdefault(name, {"us": 0.0, "calls": 0})
        rec["us"] += e_prev.elapsed_time(e) * 1e3
        rec["calls"] += 1
        e_prev = e
    for rec in per_call.values():
        rec["us"] = round(rec["us"], 2)
    say("call-by-call step done")

    # ---- each layer's attention call alone (the attention kernel and its
    # combine), cold: the Infinity Cache is evicted before every call and one
    # event pair on the stream brackets the call; the GPU is first held busy
    # so that the host queues every call ahead of it
    def attn_call(l):
        src = eng.selection_layer(l)
        kl = wl.kv_layer(l)
        args = (eng.kv_fp4[kl], eng.kv_scale[kl], eng.row_off, eng.lens, eng.max_len,
                eng.sel_pos[src], eng.sel_len[src], wl.k, wl.window)
        if blk:
            csa2.sparse_attn_decode_block(static["attn_q"][l], *args, wl.block_shared,
                                          wl.sm_scale, eng.out[l], eng.lse[l], eng.ws_attn,
                                          stream)
        else:
            csa2.sparse_attn_decode(static["attn_q"][l], *args, wl.sm_scale, eng.out[l],
                                    eng.lse[l], eng.ws_attn, stream)

    attn_reps = 3
    attn_ev = []
    with torch.cuda.stream(stream):
        torch.cuda._sleep(50_000_000)
        for _ in range(attn_reps):
            for l in range(wl.n_layers):
                evict()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                attn_call(l)
                e1.record()
                attn_ev.append((e0, e1))
    torch.cuda.synchronize()
    attn_call_us = statistics.mean(a.elapsed_time(b) for a, b in attn_ev) * 1e3
    say("attention call %.2f us (cold)" % attn_call_us)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        eng.run_step(static)
    torch.cuda.synchronize()

    # ---- timed region(s): K steps per mode ---------------------------------
    results = {}
    first_timed_step = None
    wall = 0.0
    for mode in modes:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        with torch.cuda.stream(stream):
            for _ in range(Wm):
                prepare()
                if mode == "cold":
                    evict()
                graph.replay()
        torch.cuda.synchronize()
        if not wl.append:
            assert torch.equal(eng.out, ref_out), "graph replay differs from the eager step"
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(K):
                st = prepare()
                if first_timed_step is None:
                    first_timed_step = st
                if mode == "cold":
                    evict()
                ev[i][0].record()
                graph.replay()
                ev[i][1].record()
        torch.cuda.synchronize()
        if mode == "cold":
            wall = time.perf_counter() - t0
        results[mode] = [a.elapsed_time(b) for a, b in ev]
        say("%s: %d steps, mean %.2f us" % (mode, K, statistics.mean(results[mode]) * 1e3))
    if wl.append:
        want = [L + next_step[0] * wl.block for L in case.lengths]
        assert eng.lens.cpu().tolist() == want, "lengths did not advance once per step"

    lengths = case.lengths_at(first_timed_step if wl.append else 0)
    unions = selection_unions(eng) if blk and not wl.block_shared else None
    ab = algorithmic_bytes(wl, lengths, unions)
    step_bytes = ab["step"]

    def summary(ms_list):
        ms = statistics.mean(ms_list)
        gbs = step_bytes / (ms * 1e-3) / 1e9
        return ms, gbs

    ms, step_gbs = summary(results["cold"])
    scan_s = scan_avg_ms * 1e-3
    scan_gbs = ab["scan_kernel"] / scan_s / 1e9
    # the scan's bound: whichever of its key bytes at the HBM peak, its int8
    # multiply-adds at the matrix-core peak and its score-rule vector
    # operations at the integer ALU peak takes longest (one token: HBM; a long
    # block of query tokens, such as a prefill chunk: the vector ALU)
    bounds = [
        {"bound": "hbm", "achieved": scan_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "t_peak": ab["scan_kernel"] / (HBM_PEAK_GBS * 1e9)},
        {"bound": "mfma", "achieved": ab["scan_ops"] / scan_s / 1e12, "peak": INT8_PEAK_TOPS,
         "unit": "TOP/s (int8)", "t_peak": ab["scan_ops"] / (INT8_PEAK_TOPS * 1e12)},
        {"bound": "alu", "achieved": ab["scan_alu_ops"] / scan_s / 1e12,
         "peak": round(ALU_PEAK_TOPS, 2), "unit": "T lane-ops/s (integer VALU)",
         "t_peak": ab["scan_alu_ops"] / (ALU_PEAK_TOPS * 1e12)},
    ]
    bounds.sort(key=lambda x: -x["t_peak"])
    for x in bounds:
        x["frac"] = round(x["achieved"] / x["peak"], 4)
        x["achieved"] = round(x["achieved"], 1)
        x["us_at_peak"] = round(x.pop("t_peak") * 1e6, 3)
    top = bounds[0]
    scan_roofline = {
        "kernel": ("full_score_block_kernel (Full-mode index scan, %d tokens)" % wl.block)
        if blk else "full_score_kernel (Full-mode index scan)",
        "bound": top["bound"], "achieved": top["achieved"], "peak": top["peak"],
        "unit": top["unit"], "frac": top["frac"],
        "traffic": None,
        "avg_launch_us": round(scan_avg_ms * 1e3, 3), "launches_timed": n_scan,
        "algorithmic_bytes_per_launch": ab["scan_kernel"],
        "algorithmic_int8_ops_per_launch": ab["scan_ops"],
        "algorithmic_alu_ops_per_launch": ab["scan_alu_ops"],
        "other_bounds": bounds[1:],
    }
    read_gbs = key_bytes / (read_avg_ms * 1e-3) / 1e9
    scan_roofline["traffic"] = (
        stale_traffic(os.path.join(ROOT, "profiles", "full_score_ctx_1m_counters.json"))
        if wl.name == "ctx_1m" else None)
    res = {
        "metric": METRIC,
        "value": round(1000.0 / ms, 2),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma index, bf16-mfma attention (fp32 accumulate), fp4 kv",
        "data": "synthetic (seeded SplitMix64): int8 keys (%s), N(0,1) bf16 queries and latent rows"
                % wl.keys,
        "config": {"workload": wl.name, "L": lengths[0] if wl.B == 1 else None,
                   "lengths_sum": sum(lengths), "batch": wl.B, "layers": wl.n_layers,
                   "pattern": wl.pattern, "P": wl.P, "k": wl.k, "window": wl.window,
                   "index_heads": wl.H, "query_heads": wl.Hq, "latent": wl.D,
                   "append": wl.append, "mode": "cold (Infinity Cache evicted before each step)",
                   "graph": True, "block": wl.block,
                   "block_selection": ("shared" if wl.block_shared else "per-token")
                   if blk else None},
        "step_ms_p10_p50_p90": [round(x, 5) for x in statistics.quantiles(results["cold"], n=10)[0::4]]
        if K >= 10 else None,
        "algorithmic_MB_per_step": round(step_bytes / 1e6, 3),
        "algorithmic_MB_by_call": {k: round(v / 1e6, 3) for k, v in ab.items()
                                   if k in ("append", "full", "select", "reindex", "attn")},
        "step_GBps": round(step_gbs, 1),
        "step_frac_of_hbm_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": scan_roofline,
        "read_ceiling": {"kernel": "csa2_stream_read (plain read of the key cache, scoring "
                                   "kernel's launch shape)",
                         "achieved": round(read_gbs, 1), "unit": "GB/s",
                         "frac": round(read_gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": key_bytes,
                         "avg_launch_us": round(read_avg_ms * 1e3, 3),
                         "scan_over_ceiling": round(scan_gbs / read_gbs, 4)},
        "attention_roofline": attention_roofline(ab, wl, attn_call_us, len(attn_ev)),
        "per_call_us": per_call,
        "per_call_note": "one eager step after the GPU was held busy, HIP events between the "
                         "library calls (kernel time plus the gaps between launches)",
        "timed_region_wall_s": round(wall, 4),
    }
    if wl.append or blk:
        # tokens decoded (or verified, for a block) per second
        res["tokens_per_s"] = round(wl.B * wl.block * 1000.0 / ms, 1)
    if "warm" in results:
        wms, wgbs = summary(results["warm"])
        res["warm"] = {"ms_per_step": round(wms, 5), "steps_per_s": round(1000.0 / wms, 2),
                       "step_GBps": round(wgbs, 1),
                       "step_frac_of_hbm_peak": round(wgbs / HBM_PEAK_GBS, 4)}
    if not args.no_session:
        say("session save / restore / replay")
        res["session"] = session_measure(eng, case, stream)
    if not args.no_cpu_baseline:
        say("oracle baseline")
        keys_np = eng.keys.cpu().numpy()
        res["cpu_baseline"] = cpu_baseline(wl, args.seed, first_timed_step if wl.append else 0,
                                           keys_np)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
