"""Seeded synthetic inputs, identical on the CPU and on the GPU.

This module holds none of the method's arithmetic: it only draws numbers.
Both the HIP path and the CPU oracle take their inputs from here.

Every value comes from SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used as a counter-based hash:
value i of a stream with key K is  mix(K + (i + 1) * GOLDEN).  The stream key
is itself derived from the seed and a tag per tensor, so any single element can
be regenerated on its own (the oracle only rebuilds the rows it reads).

Distributions:
  * uniform integers in [lo, hi]: top 31 bits of the hash, modulo the range;
  * N(0, 1) as bf16: a 65,536-entry table of the normal quantiles
    Phi^-1((i + 0.5) / 65536) (Python's ``statistics.NormalDist``), rounded to
    fp32 and then to bf16, indexed by 16 hash bits (four values per hash);
  * N(0, sigma) as int8: the same quantiles times sigma, rounded half-to-even
    and clipped to [-127, 127].

torch integer arithmetic wraps modulo 2^64 for int64 on both devices, which is
what the hash needs; ``splitmix64_py`` is the plain-integer definition the
tests compare against.
"""
from __future__ import annotations

import functools
import math
import statistics

import numpy as np
import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# stream tags
TAG_KEYS = 0x4B455953
TAG_PLANT = 0x504C4E54
TAG_IDXQ = 0x49445851
TAG_IDXW = 0x49445857
TAG_ATTQ = 0x41545451
TAG_KV = 0x4B565256
TAG_LEN = 0x4C454E53
TAG_RAW = 0x52415742


def splitmix64_py(x: int) -> int:
    """One SplitMix64 output for state x (plain Python integers)."""
    z = (x + GOLDEN) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, *parts: int) -> int:
    k = splitmix64_py(int(seed) & MASK64)
    for p in parts:
        k = splitmix64_py(k ^ (int(p) & MASK64))
    return k


def _s64(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >> 63 else x


def _srl(t: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor."""
    return (t >> s) & ((1 << (64 - s)) - 1)


def hash_stream(key: int, idx: torch.Tensor) -> torch.Tensor:
    """int64 tensor of SplitMix64 outputs mix(key + (idx + 1) * GOLDEN)."""
    z = idx.to(torch.int64) * _s64(GOLDEN) + _s64(key + GOLDEN)
    z = (z ^ _srl(z, 30)) * _s64(MIX1)
    z = (z ^ _srl(z, 27)) * _s64(MIX2)
    return z ^ _srl(z, 31)


def uniform_int(key: int, idx: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    h = hash_stream(key, idx)
    return (_srl(h, 33) % (hi - lo + 1) + lo)


@functools.lru_cache(maxsize=None)
def _normal_quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)], dtype=np.float64)


@functools.lru_cache(maxsize=None)
def _bf16_table_cpu() -> torch.Tensor:
    t = torch.from_numpy(_normal_quantiles()).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16)


@functools.lru_cache(maxsize=None)
def _int8_table_cpu(sigma: float) -> torch.Tensor:
    v = np.clip(np.round(sigma * _normal_quantiles()), -127, 127).astype(np.int8)
    return torch.from_numpy(v)


_table_cache: dict = {}


def _on(dev, name, fn):
    key = (name, str(dev))
    t = _table_cache.get(key)
    if t is None:
        t = fn().to(dev)
        _table_cache[key] = t
    return t


def bf16_normal(key: int, first: int, count: int, device) -> torch.Tensor:
    """``count`` N(0,1) bf16 values, elements first .. first+count-1 of the
    stream (four per hash: element e uses 16-bit field e % 4 of hash e // 4)."""
    dev = torch.device(device)
    table = _on(dev, "bf16", _bf16_table_cpu)
    e = torch.arange(first, first + count, dtype=torch.int64, device=dev)
    h = hash_stream(key, e >> 2)
    idx = (h >> ((e & 3) * 16)) & 0xFFFF
    return table[idx].view(torch.bfloat16)


def int8_normal(key: int, first: int, count: int, sigma: float, device) -> torch.Tensor:
    dev = torch.device(device)
    table = _on(dev, "i8_%g" % sigma, lambda: _int8_table_cpu(sigma))
    e = torch.arange(first, first + count, dtype=torch.int64, device=dev)
    h = hash_stream(key, e >> 2)
    idx = (h >> ((e & 3) * 16)) & 0xFFFF
    return table[idx]


def int8_uniform(key: int, first: int, count: int, device, lo: int = -127, hi: int = 127) -> torch.Tensor:
    dev = torch.device(device)
    e = torch.arange(first, first + count, dtype=torch.int64, device=dev)
    return uniform_int(key, e, lo, hi).to(torch.int8)


def uniform01(key: int, idx: torch.Tensor) -> torch.Tensor:
    """float64 in [0, 1) from the top 53 bits."""
    h = hash_stream(key, idx)
    return _srl(h, 11).to(torch.float64) * (1.0 / (1 << 53))
