"""One CSA2 decode step as an ordered sequence of C-ABI calls.

Host orchestration only: device buffers come from torch, every computation is
a libcsa2 kernel.  The layer loop follows the pages' mode split ("DeepSeek
V4.1-Flash 552B runs like 16B (CED)", "Act 2"): a Full layer scores the whole
context into a pool and selects from it, a Reindex layer re-scores the most
recent Full layer's pool, a Reuse layer attends with the most recent
selection.  Every layer then attends over its selection plus the window.
With appends, the new token's FP4 rows (every layer) and index key are written
first and the lengths advance, so the token attends to itself.
"""
from __future__ import annotations

import torch

from . import csa2
from .workloads import KV_POOL_ROWS, Case


class Engine:
    """Device-resident caches, buffers and workspaces of one workload."""

    def __init__(self, case: Case, device="cuda"):
        self.case = case
        wl = self.wl = case.wl
        dev = self.device = torch.device(device)
        self.pattern = wl.pattern
        self.keys = case.keys_all(dev)
        R = self.rows = case.total_rows
        self.kv_fp4 = torch.empty((wl.n_layers, R, wl.D // 2), dtype=torch.uint8, device=dev)
        self.kv_scale = torch.empty((wl.n_layers, R, wl.D // 32), dtype=torch.uint8, device=dev)
        self.row_off = torch.tensor(case.row_off, dtype=torch.int64, device=dev)
        self.lens = torch.tensor(case.lengths, dtype=torch.int32, device=dev)
        self.max_len = max(case.caps)
        self.total_len = sum(case.caps)
        self._fill_kv()
        B, P, k = wl.B, wl.P, wl.k
        i32 = dict(dtype=torch.int32, device=dev)
        self.pool_pos = torch.full((B, P), -7, **i32)
        self.pool_score = torch.full((B, P), -7, **i32)
        self.pool_len = torch.zeros(B, **i32)
        self.rscore = torch.full((wl.n_layers, B, P), -7, **i32)
        self.sel_pos = torch.full((wl.n_layers, B, k), -7, **i32)
        self.sel_len = torch.zeros((wl.n_layers, B), **i32)
        self.out = torch.zeros((wl.n_layers, B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((wl.n_layers, B, wl.Hq), dtype=torch.float32, device=dev)
        self.ws_full = csa2.workspace(csa2.workspace_bytes(
            csa2.OP_INDEX_FULL, B, self.max_len, self.total_len, wl.H, P, wl.k), dev)
        self.ws_attn = csa2.workspace(csa2.workspace_bytes(
            csa2.OP_SPARSE_ATTN, B, self.max_len, 0, 0, 0, k, wl.Hq, wl.D, wl.window), dev)

    # ---- cache fill (set-up, not part of a step) --------------------------
    def _fill_kv(self, chunk_rows: int = 1 << 16):
        case, wl = self.case, self.wl
        fp4 = self.kv_fp4.view(-1, wl.D // 2)
        sc = self.kv_scale.view(-1, wl.D // 32)
        n_needed = wl.n_layers * sum(case.lengths)
        direct = n_needed < KV_POOL_ROWS // 4
        if not direct:   # quantise the whole pool once, then gather rows
            pool_fp4 = torch.empty((KV_POOL_ROWS, wl.D // 2), dtype=torch.uint8, device=self.device)
            pool_sc = torch.empty((KV_POOL_ROWS, wl.D // 32), dtype=torch.uint8, device=self.device)
            for first in range(0, KV_POOL_ROWS, chunk_rows):
                n = min(chunk_rows, KV_POOL_ROWS - first)
                x = case.kv_pool_range(first, n, self.device)
                dst = torch.arange(first, first + n, dtype=torch.int64, device=self.device)
                csa2.kv_append_fp4(x, dst, pool_fp4, pool_sc)
        for layer in range(wl.n_layers):
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
            pos = [L + step for L in case.lengths]
            xs, dst = [], []
            for l in range(wl.n_layers):
                for b in range(wl.B):
                    xs.append(case.kv_bf16(l, b, [pos[b]]))
                    dst.append(l * self.rows + int(case.row_off[b]) + pos[b])
            inp["app_x"] = torch.cat(xs).to(self.device).contiguous()
            inp["app_dst"] = torch.tensor(dst, dtype=torch.int64, device=self.device)
            krow = [int(case.row_off[b]) + pos[b] for b in range(wl.B)]
            inp["key_idx"] = torch.tensor(krow, dtype=torch.int64, device=self.device)
            inp["key_rows"] = torch.stack([case.key_row(b, pos[b]) for b in range(wl.B)]).to(self.device)
        return inp

    # ---- one step -------------------------------------------------------------
    def run_step(self, inp: dict, stream=None):
        wl = self.wl
        s = stream
        if wl.append:
            csa2.kv_append_fp4(inp["app_x"], inp["app_dst"], self.kv_fp4.view(-1, wl.D // 2),
                               self.kv_scale.view(-1, wl.D // 32), s)
            self.keys.index_copy_(0, inp["key_idx"], inp["key_rows"])
            self.lens += 1
        src = None
        for l, kind in enumerate(self.pattern):
            if kind == "F":
                csa2.index_full(inp["idx_q"][l], inp["idx_w"][l], self.keys, self.row_off,
                                self.lens, self.max_len, self.total_len, wl.window, wl.P,
                                self.pool_pos, self.pool_score, self.pool_len, self.ws_full, s,
                                k=wl.k, sel_pos=self.sel_pos[l], sel_len=self.sel_len[l])
                src = l
            elif kind == "R":
                csa2.index_reindex(inp["idx_q"][l], inp["idx_w"][l], self.keys, self.row_off,
                                   self.pool_pos, self.pool_len, self.rscore[l], s)
                csa2.select_topk(self.rscore[l], self.pool_pos, self.pool_len, wl.k,
                                 self.sel_pos[l], self.sel_len[l], None, s)
                src = l
            csa2.sparse_attn_decode(inp["attn_q"][l], self.kv_fp4[l], self.kv_scale[l],
                                    self.row_off, self.lens, self.max_len, self.sel_pos[src],
                                    self.sel_len[src], wl.k, wl.window, wl.sm_scale,
                                    self.out[l], self.lse[l], self.ws_attn, s)
        return src

    def selection_layer(self, l: int) -> int:
        """Layer whose selection layer l attends with."""
        while self.pattern[l] == "U":
            l -= 1
        return l
