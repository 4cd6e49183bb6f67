"""Seeded per-step rows of the decode-loop workload (Llama3-8B-shaped, 16,384 steps).

At every decode step each (sequence, layer, KV head) unit appends one key row
and one value row, and each of its G query heads one query row. Keys follow
the repeated-segment recipe of the other workloads, laid out along time: a
step inside a copy run takes the fresh key of an earlier step (at most
``max_back`` steps back) plus N(0, sigma^2) noise; run positions are per
sequence and shared by its layers and heads. Values and queries are i.i.d.
N(0, 1).

Rows are computed from counters, not drawn from a stateful generator: every
element is a hash of (seed, stream, unit, step, element), turned into a
normal variate by Box-Muller. Any step's rows, including the fresh key of a
copy source, can be regenerated on its own, on any device, without history.
Nothing here scores, selects or moves rows.
"""
from __future__ import annotations

import math

import numpy as np

from .gen import HEAD_DIM, segment_layout

_M32 = 0xFFFFFFFF
# stream ids of the independent variates
_BASE, _NOISE, _VALUE, _QUERY = 1, 2, 3, 4


def _hash32(x):
    """32-bit integer finaliser (xor-shift / multiply rounds) on int64 tensors
    holding values in [0, 2^32)."""
    x = x & _M32
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & _M32
    x = x ^ (x >> 16)
    return x


def _normals(key, n: int):
    """n standard normal variates per entry of the int64 tensor `key` [...]:
    returns float32 [..., n]."""
    import torch
    j = torch.arange(n, device=key.device, dtype=torch.int64)
    h = _hash32(key[..., None] * 0x9E3779B1 + j)          # [..., n]
    h1 = _hash32(h ^ 0x68E31DA4)
    h2 = _hash32(h ^ 0x1B56C4E9)
    u1 = ((h1 >> 8).to(torch.float32) + 0.5) * (1.0 / 16777216.0)   # (0, 1)
    u2 = (h2 >> 8).to(torch.float32) * (1.0 / 16777216.0)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


class DecodeStream:
    """Rows of step t for every unit (ordered (sequence, layer, KV head))."""

    def __init__(self, seed: int, batch: int, layers: int, kv_heads: int, gqa: int, steps: int,
                 coverage: float = 0.40, sigma: float = 0.02, max_back: int = 1024,
                 dtype: str = "bf16", device: str = "cuda"):
        import torch
        self.seed, self.batch, self.gqa, self.steps = seed, batch, gqa, steps
        self.hps = layers * kv_heads
        self.units = batch * self.hps
        self.sigma = sigma
        self.device = device
        self.dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        rng = np.random.Generator(np.random.PCG64(seed))
        layouts = np.stack([segment_layout(rng, steps, coverage, max_back=max_back)
                            for _ in range(batch)])
        self.layouts = layouts                                   # [batch, steps], -1 = fresh
        self.coverage = float((layouts >= 0).mean())
        self._lay = torch.as_tensor(layouts, device=device)
        self._seq = torch.arange(self.units, device=device) // self.hps
        self._unit = torch.arange(self.units, device=device, dtype=torch.int64)

    def _key(self, stream: int, step):
        """int64 [units] counter keys for (stream, unit, step); step [units] or int."""
        h = _hash32(self._unit * 0x01000193 + (self.seed * 0x9E3779B1 + stream * 0x85EBCA77))
        return _hash32(h ^ _hash32(step * 0xC2B2AE3D + 0x27D4EB2F))

    def rows(self, t: int):
        """(k [units, 128], v [units, 128], q [units, G, 128]) of step t."""
        import torch
        src = self._lay[self._seq, t]                            # [units]
        rep = src >= 0
        t_base = torch.where(rep, src, torch.full_like(src, t)).to(torch.int64)
        k = _normals(self._key(_BASE, t_base), HEAD_DIM)
        noise = _normals(self._key(_NOISE, torch.full_like(t_base, t)), HEAD_DIM)
        k = torch.where(rep[:, None], k + self.sigma * noise, k)
        v = _normals(self._key(_VALUE, torch.full_like(t_base, t)), HEAD_DIM)
        q = _normals(self._key(_QUERY, torch.full_like(t_base, t)), self.gqa * HEAD_DIM)
        return (k.to(self.dtype), v.to(self.dtype),
                q.view(self.units, self.gqa, HEAD_DIM).to(self.dtype))
