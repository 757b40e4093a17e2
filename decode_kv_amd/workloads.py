"""The synthetic decode workloads and their seeded inputs.

The workloads, named by what they are:

  tiny_4k       L=4,096, 1 sequence, one Full layer (P=1,024, k=64), 4 index
                heads, 16 query heads; uniform int8 keys + 8 planted keys.
  single_64k    L=65,536, 1 sequence, one Full layer (P=16,384, k=512), 64
                index heads, 64 query heads; N(0,30) int8 keys with 256
                planted clusters of 8.
  batch8_256k   L=262,144, 8 sequences, layers F R U U, one FP4 append per
                sequence and layer per step, 64 steps.
  ctx_1m        L=1,048,576, 1 sequence, 20 layers F R U U R U U U R ...;
                N(0,30) int8 keys with 1,024 planted keys at log-uniform
                distance from the end.
  ragged32_1m   32 sequences, lengths log-uniform in [4,096, 1,048,576], the
                20-layer pattern, one append per sequence and layer per step,
                64 steps, queries re-drawn every step.
  ctx_1m_shared, ragged32_1m_shared
                the same with one FP4 latent cache shared by all 20 layers
                (one append per sequence per step).
  ctx_1m_block5, batch8_256k_block5 (and *_shared)
                verify blocks of 5 tokens per sequence: ctx_1m verifying its
                last 5 cached positions, batch8_256k appending and verifying 5
                tokens per sequence and step; per-token or shared selection.
  prefill_128k_chunk256
                chunked prefill indexing: the last 256 positions of a 131,072
                token prompt score their own causal prefixes (one Full layer,
                per-token pools and selections, then attention).

Everywhere: window 128, index key dim 64, latent dim 512, softmax scale
1/sqrt(512).  Nothing here computes any part of the method; the only
arithmetic is the generation recipe (see the module docstring of
:mod:`decode_kv_amd.inputs`).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

from . import inputs as I


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: Optional[int]                       # fixed initial length of every sequence
    len_range: Optional[Tuple[int, int]]   # or log-uniform lengths in [lo, hi]
    n_layers: int
    P: int
    k: int
    window: int
    H: int
    Hq: int
    keys: str                              # "uniform8" | "clusters" | "planted"
    n_planted: int
    steps: int
    append: bool
    redraw_queries: bool
    shared_kv: bool = False                # one FP4 latent cache read by every layer
    block: int = 1                         # tokens verified per step (a drafted block)
    block_shared: bool = False             # the block's tokens share one pool / selection
    Dk: int = 64
    D: int = 512

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def pattern(self) -> str:
        return "".join(layer_kind(l) for l in range(self.n_layers))

    @property
    def n_kv(self) -> int:
        """FP4 latent caches: one per layer, or one for all layers."""
        return 1 if self.shared_kv else self.n_layers

    def kv_layer(self, l: int) -> int:
        """Cache that layer l attends to."""
        return 0 if self.shared_kv else l

    @property
    def n_lists(self) -> int:
        """Pools / selections per step: one per sequence, or one per token
        of a block whose tokens select on their own."""
        return self.B if self.block == 1 or self.block_shared else self.B * self.block

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def layer_kind(l: int) -> str:
    """F at layer 0, R at layer 1 and at every layer divisible by 4, U else."""
    return "F" if l == 0 else ("R" if (l == 1 or l % 4 == 0) else "U")


WORKLOADS = {
    "tiny_4k": Workload("tiny_4k", B=1, L=4096, len_range=None, n_layers=1, P=1024, k=64,
                        window=128, H=4, Hq=16, keys="uniform8", n_planted=8, steps=1,
                        append=False, redraw_queries=False),
    "single_64k": Workload("single_64k", B=1, L=65536, len_range=None, n_layers=1, P=16384,
                           k=512, window=128, H=64, Hq=64, keys="clusters", n_planted=2048,
                           steps=1, append=False, redraw_queries=False),
    "batch8_256k": Workload("batch8_256k", B=8, L=262144, len_range=None, n_layers=4,
                            P=16384, k=512, window=128, H=64, Hq=64, keys="planted",
                            n_planted=1024, steps=64, append=True, redraw_queries=True),
    "ctx_1m": Workload("ctx_1m", B=1, L=1048576, len_range=None, n_layers=20, P=16384,
                       k=512, window=128, H=64, Hq=64, keys="planted", n_planted=1024,
                       steps=1, append=False, redraw_queries=False),
    "ragged32_1m": Workload("ragged32_1m", B=32, L=None, len_range=(4096, 1048576),
                            n_layers=20, P=16384, k=512, window=128, H=64, Hq=64,
                            keys="planted", n_planted=1024, steps=64, append=True,
                            redraw_queries=True),
}
# The shared-KV variants: every decoder layer attends to one FP4 latent cache
# (the pages' setting in which only some layers build global KV and the
# others reuse it), so a decode step appends one FP4 row per sequence.
WORKLOADS["ctx_1m_shared"] = WORKLOADS["ctx_1m"].scaled(name="ctx_1m_shared", shared_kv=True)
WORKLOADS["ragged32_1m_shared"] = WORKLOADS["ragged32_1m"].scaled(name="ragged32_1m_shared",
                                                                  shared_kv=True)
# Verify blocks: five drafted tokens checked in one step, each token with its
# own pool and selection, or one shared by the block (the pages give the block
# size, not how its tokens share the selection).  The block's tokens are the
# last five cached positions; the batched variant appends five tokens per
# sequence and step before verifying them.
WORKLOADS["ctx_1m_block5"] = WORKLOADS["ctx_1m"].scaled(name="ctx_1m_block5", block=5)
WORKLOADS["ctx_1m_block5_shared"] = WORKLOADS["ctx_1m"].scaled(name="ctx_1m_block5_shared",
                                                               block=5, block_shared=True)
WORKLOADS["batch8_256k_block5"] = WORKLOADS["batch8_256k"].scaled(name="batch8_256k_block5",
                                                                  block=5)
WORKLOADS["batch8_256k_block5_shared"] = WORKLOADS["batch8_256k"].scaled(
    name="batch8_256k_block5_shared", block=5, block_shared=True)
# Chunked prefill indexing: the last 256 tokens of a 131,072-token prompt,
# already in the cache, each rank their own causal prefix (per-token pool and
# selection) in one Full layer, then attend.
WORKLOADS["prefill_128k_chunk256"] = Workload(
    "prefill_128k_chunk256", B=1, L=131072, len_range=None, n_layers=1, P=16384, k=512,
    window=128, H=64, Hq=64, keys="planted", n_planted=1024, steps=1, append=False,
    redraw_queries=False, block=256)


KV_POOL_ROWS = 1 << 20


class Case:
    """Seeded inputs of one workload.  Device-agnostic: the same (workload,
    seed) gives bit-identical tensors on the CPU and on the GPU."""

    def __init__(self, wl: Workload, seed: int = 0, device="cpu"):
        self.wl = wl
        self.seed = int(seed)
        self.device = torch.device(device)
        self.lengths = self._lengths()
        extra = wl.steps * wl.block if wl.append else 0
        self.caps = [L + extra for L in self.lengths]
        offs = np.zeros(wl.B, dtype=np.int64)
        if wl.B > 1:
            offs[1:] = np.cumsum(self.caps)[:-1]
        self.row_off = offs
        self.total_rows = int(sum(self.caps))

    # ---- lengths -------------------------------------------------------
    def _lengths(self):
        wl = self.wl
        if wl.L is not None:
            return [int(wl.L)] * wl.B
        lo, hi = wl.len_range
        u = I.uniform01(I.stream_key(self.seed, I.TAG_LEN), torch.arange(wl.B))
        L = torch.floor(torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
        return [int(min(hi, max(lo, x))) for x in L.tolist()]

    def lengths_at(self, step: int):
        """Cached lengths seen by the layers of decode step `step` (the step's
        appends, one token or a block of them, happen before the layers run)."""
        wl = self.wl
        return [L + ((step + 1) * wl.block if wl.append else 0) for L in self.lengths]

    def _qkey(self, tag: int, step: int, layer: int, b: int, t: int) -> int:
        wl = self.wl
        st = step if wl.redraw_queries else 0
        if wl.block == 1:
            return I.stream_key(self.seed, tag, st, layer, b)
        return I.stream_key(self.seed, tag, st, layer, b, t)

    # ---- index queries / weights (token t of a block) ----------------------
    def index_q(self, step: int, layer: int, b: int, t: int = 0) -> torch.Tensor:
        wl = self.wl
        key = self._qkey(I.TAG_IDXQ, step, layer, b, t)
        return I.int8_uniform(key, 0, wl.H * wl.Dk, self.device).view(wl.H, wl.Dk)

    def index_w(self, step: int, layer: int, b: int, t: int = 0) -> torch.Tensor:
        wl = self.wl
        key = self._qkey(I.TAG_IDXW, step, layer, b, t)
        return I.int8_uniform(key, 0, wl.H, self.device, 0, 15)

    def index_qw_batch(self, step: int, layer: int):
        """[B][H][Dk] and [B][H]; with blocks [B][T][H][Dk] and [B][T][H]."""
        wl = self.wl
        if wl.block == 1:
            q = torch.stack([self.index_q(step, layer, b) for b in range(wl.B)])
            w = torch.stack([self.index_w(step, layer, b) for b in range(wl.B)])
        else:
            q = torch.stack([torch.stack([self.index_q(step, layer, b, t) for t in range(wl.block)])
                             for b in range(wl.B)])
            w = torch.stack([torch.stack([self.index_w(step, layer, b, t) for t in range(wl.block)])
                             for b in range(wl.B)])
        return q.contiguous(), w.contiguous()

    # ---- attention queries ---------------------------------------------
    def attn_q(self, step: int, layer: int, b: int, t: int = 0) -> torch.Tensor:
        wl = self.wl
        key = self._qkey(I.TAG_ATTQ, step, layer, b, t)
        return I.bf16_normal(key, 0, wl.Hq * wl.D, self.device).view(wl.Hq, wl.D)

    def attn_q_batch(self, step: int, layer: int) -> torch.Tensor:
        """[B][Hq][D]; with blocks [B][T][Hq][D]."""
        wl = self.wl
        if wl.block == 1:
            return torch.stack([self.attn_q(step, layer, b) for b in range(wl.B)]).contiguous()
        return torch.stack([torch.stack([self.attn_q(step, layer, b, t) for t in range(wl.block)])
                            for b in range(wl.B)]).contiguous()

    # ---- latent KV rows (bf16, before quantisation) ----------------------
    # The latent row of (layer, sequence, position) is row `kv_row_id` of a
    # pool of KV_POOL_ROWS seeded N(0,1) rows: generating every element of a
    # 20-layer, multi-million-token cache by hashing would dominate set-up, and
    # a pool of 2^20 rows keeps repeats inside one attended set rare.
    def kv_row_id(self, layer: int, b: int, positions) -> torch.Tensor:
        pos = torch.as_tensor(positions, dtype=torch.int64, device=self.device).reshape(-1)
        key = I.stream_key(self.seed, I.TAG_KV, self.wl.kv_layer(layer), b)
        return I._srl(I.hash_stream(key, pos), 44)           # top 20 bits

    def kv_pool_rows(self, row_ids, device=None) -> torch.Tensor:
        """bf16 rows of the pool, [n, D]."""
        dev = torch.device(device) if device is not None else self.device
        D = self.wl.D
        rid = torch.as_tensor(row_ids, dtype=torch.int64, device=dev).reshape(-1)
        key = I.stream_key(self.seed, I.TAG_KV, 0xFFFF)
        table = I._on(dev, "bf16", I._bf16_table_cpu)
        e = rid[:, None] * D + torch.arange(D, dtype=torch.int64, device=dev)[None, :]
        h = I.hash_stream(key, e >> 2)
        idx = (h >> ((e & 3) * 16)) & 0xFFFF
        return table[idx].view(torch.bfloat16)

    def kv_pool_range(self, first: int, count: int, device=None) -> torch.Tensor:
        dev = torch.device(device) if device is not None else self.device
        key = I.stream_key(self.seed, I.TAG_KV, 0xFFFF)
        D = self.wl.D
        return I.bf16_normal(key, first * D, count * D, dev).view(count, D)

    def kv_bf16(self, layer: int, b: int, positions) -> torch.Tensor:
        """bf16 latent rows of layer `layer`, sequence b, at `positions`."""
        return self.kv_pool_rows(self.kv_row_id(layer, b, positions))

    # ---- index keys ------------------------------------------------------
    def aligned_vector(self, b: int) -> np.ndarray:
        """Key most aligned with layer 0's step-0 index query of sequence b:
        u = sum_h w_h q_h, a = round(127 u / max|u|) (half to even)."""
        q = self.index_q(0, 0, b).cpu().numpy().astype(np.float64)
        w = self.index_w(0, 0, b).cpu().numpy().astype(np.float64)
        u = (w[:, None] * q).sum(axis=0)
        m = np.abs(u).max()
        if m == 0:
            return np.zeros(self.wl.Dk, dtype=np.int8)
        return np.clip(np.round(127.0 * u / m), -127, 127).astype(np.int8)

    def _noise(self, tag: int, b: int, count: int, sigma: float) -> np.ndarray:
        key = I.stream_key(self.seed, I.TAG_PLANT, tag, b)
        return I.int8_normal(key, 0, count, sigma, "cpu").numpy().astype(np.int32)

    def _distinct_positions(self, b: int, tag: int, E: int, n: int, log_distance: bool):
        """n distinct eligible positions in [0, E): uniform (hash order of all
        positions) or at log-uniform distance from the end of the context."""
        n = min(n, E)
        if n <= 0:
            return np.zeros(0, dtype=np.int64)
        key = I.stream_key(self.seed, I.TAG_PLANT, tag, b, 7)
        if not log_distance:
            h = I.hash_stream(key, torch.arange(E, dtype=torch.int64))
            return torch.argsort(h, stable=True)[:n].numpy().astype(np.int64)
        if n == E:
            # every eligible position is planted (a short sequence); the draw
            # below never reaches distance L, i.e. position 0
            return np.arange(E, dtype=np.int64)
        W = self.wl.window
        L = E + W
        out, seen, i = [], set(), 0
        lo, hi = math.log(W + 1), math.log(L)
        while len(out) < n:
            if i > 4 * n * 100_000:
                raise RuntimeError("planted positions: draw did not finish")
            u = I.uniform01(key, torch.arange(i, i + 4 * n, dtype=torch.int64)).numpy()
            i += 4 * n
            d = np.floor(np.exp(lo + u * (hi - lo))).astype(np.int64)
            for dd in d:
                p = int(L - dd)
                if 0 <= p < E and p not in seen:
                    seen.add(p)
                    out.append(p)
                    if len(out) == n:
                        break
        return np.array(out, dtype=np.int64)

    def planted(self, b: int):
        """(positions, key rows) planted into sequence b's index keys."""
        wl = self.wl
        L = self.lengths[b]
        E = max(0, L - wl.window)
        a = self.aligned_vector(b).astype(np.int32)
        if wl.keys == "uniform8":
            pos = self._distinct_positions(b, 1, E, wl.n_planted, False)
            rows = np.repeat(a[None, :], len(pos), axis=0)
        elif wl.keys == "clusters":
            pos = self._distinct_positions(b, 2, E, wl.n_planted, False)
            n_cl = max(1, wl.n_planted // 8)
            alpha = 0.35 + 0.65 * np.arange(n_cl) / max(1, n_cl - 1)
            cn = self._noise(3, b, n_cl * wl.Dk, 8.0).reshape(n_cl, wl.Dk)
            centres = np.clip(np.round(alpha[:, None] * a[None, :]) + cn, -127, 127)
            mn = self._noise(4, b, len(pos) * wl.Dk, 4.0).reshape(len(pos), wl.Dk)
            rows = np.clip(centres[np.arange(len(pos)) // 8 % n_cl] + mn, -127, 127)
        else:
            pos = self._distinct_positions(b, 5, E, wl.n_planted, True)
            mn = self._noise(6, b, len(pos) * wl.Dk, 4.0).reshape(len(pos), wl.Dk)
            rows = np.clip(a[None, :] + mn, -127, 127)
        return pos, rows.astype(np.int8)

    def keys_seq(self, b: int, device=None) -> torch.Tensor:
        """Index keys of sequence b, all `caps[b]` rows, [cap, Dk] int8."""
        dev = torch.device(device) if device is not None else self.device
        wl = self.wl
        cap = self.caps[b]
        key = I.stream_key(self.seed, I.TAG_KEYS, b)
        if wl.keys == "uniform8":
            k = I.int8_uniform(key, 0, cap * wl.Dk, dev)
        else:
            k = I.int8_normal(key, 0, cap * wl.Dk, 30.0, dev)
        k = k.view(cap, wl.Dk)
        pos, rows = self.planted(b)
        if len(pos):
            k[torch.as_tensor(pos, device=dev)] = torch.as_tensor(rows, device=dev)
        return k

    def key_row(self, b: int, pos: int, device=None) -> torch.Tensor:
        """Index key of sequence b at a position that was not planted (the
        base distribution), e.g. a token appended during decode."""
        dev = torch.device(device) if device is not None else self.device
        wl = self.wl
        key = I.stream_key(self.seed, I.TAG_KEYS, b)
        if wl.keys == "uniform8":
            return I.int8_uniform(key, pos * wl.Dk, wl.Dk, dev)
        return I.int8_normal(key, pos * wl.Dk, wl.Dk, 30.0, dev)

    def keys_all(self, device=None) -> torch.Tensor:
        dev = torch.device(device) if device is not None else self.device
        out = torch.empty((self.total_rows, self.wl.Dk), dtype=torch.int8, device=dev)
        for b in range(self.wl.B):
            o = int(self.row_off[b])
            out[o:o + self.caps[b]] = self.keys_seq(b, dev)
        return out


def raw_fp4_rows(seed: int, n: int, D: int, scale_lo: int, scale_hi: int, device="cpu"):
    """Arbitrary FP4 bytes (every code) with scale bytes uniform in
    [scale_lo, scale_hi]: for edge-case tests of the dequantising reader."""
    key = I.stream_key(seed, I.TAG_RAW, 1)
    codes = I.uniform_int(key, torch.arange(n * D // 2, device=device), 0, 255)
    codes = codes.to(torch.uint8).view(n, D // 2)
    key2 = I.stream_key(seed, I.TAG_RAW, 2)
    scales = I.uniform_int(key2, torch.arange(n * (D // 32), device=device), scale_lo, scale_hi)
    return codes.contiguous(), scales.to(torch.uint8).view(n, D // 32).contiguous()
