"""One CSA2 decode step as an ordered sequence of C-ABI calls.

Host orchestration only: device buffers come from torch, every computation is
a libcsa2 kernel.  The layer loop follows the pages' mode split ("DeepSeek
V4.1-Flash 552B runs like 16B (CED)", "Act 2"): a Full layer scores the whole
context into a pool and selects from it, a Reindex layer re-scores the most
recent Full layer's pool, a Reuse layer attends with the most recent
selection.  Every layer then attends over its selection plus the window.
With appends, one library call first writes the new token's FP4 rows (every
layer) and index key at the device-side length and advances it, so the token
attends to itself.  A verify block of T drafted tokens per sequence appends
its T tokens (one call) and runs the block variants of the calls, which
score, select and attend for all T tokens at once.
"""
from __future__ import annotations

import torch

from . import csa2
from .workloads import KV_POOL_ROWS, Case


def copy_inputs(dst: dict, src: dict, stream=None):
    """Copy one step's inputs (as returned by Engine.step_inputs) into the
    buffers of another, e.g. the static inputs of a captured step."""
    ctx = torch.cuda.stream(stream) if stream is not None else None
    if ctx is not None:
        ctx.__enter__()
    try:
        for key, v in src.items():
            if isinstance(v, dict):
                for l, t in v.items():
                    dst[key][l].copy_(t, non_blocking=True)
            elif isinstance(v, list):
                for a, t in zip(dst[key], v):
                    a.copy_(t, non_blocking=True)
            else:
                dst[key].copy_(v, non_blocking=True)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


class Engine:
    """Device-resident caches, buffers and workspaces of one workload."""

    def __init__(self, case: Case, device="cuda"):
        self.case = case
        wl = self.wl = case.wl
        dev = self.device = torch.device(device)
        self.pattern = wl.pattern
        self.keys = case.keys_all(dev)
        R = self.rows = case.total_rows
        self.kv_fp4 = torch.empty((wl.n_kv, R, wl.D // 2), dtype=torch.uint8, device=dev)
        self.kv_scale = torch.empty((wl.n_kv, R, wl.D // 32), dtype=torch.uint8, device=dev)
        self.row_off = torch.tensor(case.row_off, dtype=torch.int64, device=dev)
        self.lens = torch.tensor(case.lengths, dtype=torch.int32, device=dev)
        self.max_len = max(case.caps)
        self.total_len = sum(case.caps)
        self._fill_kv()
        B, P, k, T = wl.B, wl.P, wl.k, wl.block
        nl = wl.n_lists                      # pools / selections: per sequence or per token
        i32 = dict(dtype=torch.int32, device=dev)
        self.pool_pos = torch.full((nl, P), -7, **i32)
        self.pool_score = torch.full((nl, P), -7, **i32)
        self.pool_len = torch.zeros(nl, **i32)
        self.rscore = torch.full((wl.n_layers, nl, P), -7, **i32)
        self.sel_pos = torch.full((wl.n_layers, nl, k), -7, **i32)
        self.sel_len = torch.zeros((wl.n_layers, nl), **i32)
        rows = (B,) if T == 1 else (B, T)   # query rows: a token per sequence, or a block
        self.out = torch.zeros((wl.n_layers, *rows, wl.Hq, wl.D), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((wl.n_layers, *rows, wl.Hq), dtype=torch.float32, device=dev)
        sh = wl.block_shared
        self.ws_full = csa2.workspace(csa2.block_workspace_bytes(
            csa2.OP_INDEX_FULL, B, T, sh, self.max_len, self.total_len, wl.H, P, wl.k), dev)
        self.ws_attn = csa2.workspace(csa2.block_workspace_bytes(
            csa2.OP_SPARSE_ATTN, B, T, sh, self.max_len, 0, 0, 0, k, wl.Hq, wl.D, wl.window), dev)

    # ---- cache fill (set-up, not part of a step) --------------------------
    def _fill_kv(self, chunk_rows: int = 1 << 16):
        case, wl = self.case, self.wl
        fp4 = self.kv_fp4.view(-1, wl.D // 2)
        sc = self.kv_scale.view(-1, wl.D // 32)
        n_needed = wl.n_kv * sum(case.lengths)
        direct = n_needed < KV_POOL_ROWS // 4
        if not direct:   # quantise the whole pool once, then gather rows
            pool_fp4 = torch.empty((KV_POOL_ROWS, wl.D // 2), dtype=torch.uint8, device=self.device)
            pool_sc = torch.empty((KV_POOL_ROWS, wl.D // 32), dtype=torch.uint8, device=self.device)
            for first in range(0, KV_POOL_ROWS, chunk_rows):
                n = min(chunk_rows, KV_POOL_ROWS - first)
                x = case.kv_pool_range(first, n, self.device)
                dst = torch.arange(first, first + n, dtype=torch.int64, device=self.device)
                csa2.kv_append_fp4(x, dst, pool_fp4, pool_sc)
        for layer in range(wl.n_kv):
            for b in range(wl.B):
                L0 = case.lengths[b]
                base = layer * self.rows + int(case.row_off[b])
                for first in range(0, L0, chunk_rows):
                    n = min(chunk_rows, L0 - first)
                    pos = torch.arange(first, first + n, dtype=torch.int64, device=self.device)
                    dst = base + pos
                    if direct:
                        csa2.kv_append_fp4(case.kv_bf16(layer, b, pos), dst, fp4, sc)
                    else:
                        ids = case.kv_row_id(layer, b, pos)
                        fp4[dst] = pool_fp4[ids]
                        sc[dst] = pool_sc[ids]
        torch.cuda.synchronize(self.device)

    # ---- per-step inputs ----------------------------------------------------
    def step_inputs(self, step: int) -> dict:
        case, wl = self.case, self.wl
        inp = {"idx_q": {}, "idx_w": {}, "attn_q": []}
        for l, kind in enumerate(self.pattern):
            if kind in "FR":
                q, w = case.index_qw_batch(step, l)
                inp["idx_q"][l], inp["idx_w"][l] = q.to(self.device), w.to(self.device)
            inp["attn_q"].append(case.attn_q_batch(step, l).to(self.device))
        if wl.append:
            # token j of step `step` sits at position L0 + step * T + j; the
            # library writes it at the device-side length, which equals that
            # position when the steps run in order
            T = wl.block
            xs, ks = [], []
            for j in range(T):
                pos = [L + step * T + j for L in case.lengths]
                xs += [case.kv_bf16(l, b, [pos[b]]) for l in range(wl.n_kv) for b in range(wl.B)]
                ks += [case.key_row(b, pos[b]) for b in range(wl.B)]
            inp["app_x"] = torch.cat(xs).view(T, wl.n_kv, wl.B, wl.D).to(self.device).contiguous()
            inp["key_rows"] = torch.stack(ks).view(T, wl.B, wl.Dk).to(self.device).contiguous()
        return inp

    # ---- one step -------------------------------------------------------------
    def run_step(self, inp: dict, stream=None, mark=None):
        """Enqueue one decode step on `stream` (torch's current stream if None).
        mark(name), when given, is called after each library call with the
        call's kind ("append", "full", "reindex", "select", "attn"); the
        benchmark records an event there to time the calls one by one."""
        wl = self.wl
        s = stream
        note = mark if mark is not None else (lambda name: None)
        if wl.append:
            if wl.block == 1:
                csa2.append_token(inp["app_x"][0], inp["key_rows"][0], self.row_off, self.lens,
                                  self.kv_fp4, self.kv_scale, self.keys, s)
            else:                            # a block's tokens in one call
                csa2.append_tokens(inp["app_x"], inp["key_rows"], self.row_off, self.lens,
                                   self.kv_fp4, self.kv_scale, self.keys, s)
            note("append")
        blk = wl.block > 1
        sh = wl.block_shared
        src = None
        for l, kind in enumerate(self.pattern):
            if kind == "F":
                full = csa2.index_full_block if blk else csa2.index_full
                extra = (sh,) if blk else ()
                full(inp["idx_q"][l], inp["idx_w"][l], self.keys, self.row_off, self.lens,
                     self.max_len, self.total_len, wl.window, wl.P, *extra, self.pool_pos,
                     self.pool_score, self.pool_len, self.ws_full, s, k=wl.k,
                     sel_pos=self.sel_pos[l], sel_len=self.sel_len[l])
                note("full")
                src = l
            elif kind == "R":
                if blk:
                    csa2.index_reindex_block(inp["idx_q"][l], inp["idx_w"][l], self.keys,
                                             self.row_off, self.pool_pos, self.pool_len, sh,
                                             self.rscore[l], s)
                else:
                    csa2.index_reindex(inp["idx_q"][l], inp["idx_w"][l], self.keys, self.row_off,
                                       self.pool_pos, self.pool_len, self.rscore[l], s)
                note("reindex")
                csa2.select_topk(self.rscore[l], self.pool_pos, self.pool_len, wl.k,
                                 self.sel_pos[l], self.sel_len[l], None, s)
                note("select")
                src = l
            kl = wl.kv_layer(l)
            args = (self.kv_fp4[kl], self.kv_scale[kl], self.row_off, self.lens, self.max_len,
                    self.sel_pos[src], self.sel_len[src], wl.k, wl.window)
            if blk:
                csa2.sparse_attn_decode_block(inp["attn_q"][l], *args, sh, wl.sm_scale,
                                              self.out[l], self.lse[l], self.ws_attn, s)
            else:
                csa2.sparse_attn_decode(inp["attn_q"][l], *args, wl.sm_scale, self.out[l],
                                        self.lse[l], self.ws_attn, s)
            note("attn")
        return src

    def selection_layer(self, l: int) -> int:
        """Layer whose selection layer l attends with."""
        while self.pattern[l] == "U":
            l -= 1
        return l
