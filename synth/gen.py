"""Seeded generators for the five synthetic workloads of the R-KV compression step.

The workloads stand in for the pages' setting (R1-distilled Llama3-8B and
Qwen-14B decoding long math chains of thought with a 1024-token budget), whose
datasets and weights are not available. What is drawn:

* keys, values and window queries, i.i.d. N(0, 1), rounded to bf16 by
  round-to-nearest-even where the workload is bf16;
* "repeated segments": runs of 16..64 tokens that copy an earlier run of the
  same head's fresh key stream plus N(0, sigma^2) noise, placed greedily until
  a target fraction of the tokens is covered. Reasoning traces restate earlier
  content, which is what the redundancy score is meant to find;
* for the tiny workload, single near-duplicate tokens instead of runs;
* for the paged workload, ragged lengths, page-rounded budgets, a shuffled
  page table and an initial free list.

Every array is reproducible from (workload, seed). Host arrays are numpy
float32 holding values that are exact in the workload's dtype; device tensors
are torch tensors in that dtype. Nothing here scores, selects or moves rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16

# The five workloads.  Sizes follow the models the pages evaluate on
# (Llama3-8B: 32 layers, 32 query heads, 8 KV heads; Qwen-14B: 48 layers,
# 40 query heads, 8 KV heads; head_dim 128) and the pages' defaults
# (kv_budget 1024, window_size 8, mix_lambda 0.1, divide_length 128).
CONFIGS = {
    0: dict(name="tiny-fp32", batch=1, layers=1, kv_heads=1, gqa=4, n=96, budget=64,
            window=8, lam=0.1, dtype="f32", dup_frac=0.30, dup_sigma=0.01),
    1: dict(name="llama3-8b-1layer", batch=1, layers=1, kv_heads=8, gqa=4, n=1152,
            budget=1024, window=8, lam=0.1, dtype="bf16", coverage=0.40, sigma=0.02),
    2: dict(name="llama3-8b-decode-event", batch=64, layers=32, kv_heads=8, gqa=4,
            n=1152, budget=1024, window=8, lam=0.1, dtype="bf16", coverage=0.40,
            sigma=0.02, divide_length=128, steps=16384),
    3: dict(name="qwen-14b", batch=32, layers=48, kv_heads=8, gqa=5, n=2176, budget=2048,
            window=8, lams=(0.0, 0.1, 1.0), dtype="bf16", coverage=0.25, sigma=0.02),
    4: dict(name="paged-ragged", seqs=128, kv_heads=8, gqa=4, n_min=2048, n_max=32768,
            frac_min=0.10, frac_max=0.34, window=8, lam=0.1, dtype="bf16",
            coverage=0.40, sigma=0.02, page_size=PAGE_SIZE, spare_pages=1024),
}


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).reshape(x.shape)


def segment_layout(rng: np.random.Generator, n: int, coverage: float, lmin: int = 16,
                   lmax: int = 64, tol: float = 0.01,
                   max_back: Optional[int] = None) -> np.ndarray:
    """Positions of repeated runs in one sequence.

    Returns ``src`` of length n: -1 for a fresh token, else the earlier
    position whose fresh key this token copies. Runs have length U{lmin..lmax},
    do not overlap one another, and copy a run that ends before they start
    (and starts at most ``max_back`` tokens earlier when given). Runs are
    placed until ``coverage`` of the tokens is reached, overshooting by at
    most ``tol``.
    """
    src = np.full(n, -1, dtype=np.int64)
    if coverage <= 0 or n < 2 * lmin:
        return src
    target = coverage * n
    cap = int(math.floor((coverage + tol) * n))
    covered = 0
    attempts = 0
    while covered < target and attempts < 100000:
        attempts += 1
        length = int(rng.integers(lmin, lmax + 1))
        length = min(length, cap - covered)
        if length < 1:
            break
        t0 = int(rng.integers(length, n - length + 1))
        if (src[t0:t0 + length] >= 0).any():
            continue
        lo = 0 if max_back is None else max(0, t0 - max_back)
        s0 = int(rng.integers(lo, t0 - length + 1))
        src[t0:t0 + length] = np.arange(s0, s0 + length)
        covered += length
    return src


def plant_near_duplicates(rng: np.random.Generator, keys: np.ndarray, frac: float,
                          sigma: float):
    """Replace round(frac*N) tokens at positions >= 1 by an earlier key plus noise.

    Works in place on ``keys`` [N, d], in increasing position order, copying
    the earlier key as it stands. Returns (positions, sources).
    """
    n, d = keys.shape
    count = int(round(frac * n))
    pos = np.sort(rng.choice(np.arange(1, n), size=count, replace=False))
    srcs = np.empty(count, dtype=np.int64)
    for k, t in enumerate(pos):
        s = int(rng.integers(0, t))
        srcs[k] = s
        keys[t] = keys[s] + sigma * rng.standard_normal(d)
    return pos, srcs


@dataclasses.dataclass
class DenseCase:
    """One dense call's inputs: K, V [Bh, N, d], Q_win [Bh, G, w, d]."""
    K: object
    V: object
    Q: object
    budget: int
    window: int
    lam: float
    dtype: str
    layouts: Optional[np.ndarray] = None   # [batch, N] run sources, or None
    heads_per_seq: int = 1
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def num_heads(self) -> int:
        return int(self.K.shape[0])

    @property
    def n(self) -> int:
        return int(self.K.shape[1])

    @property
    def gqa(self) -> int:
        return int(self.Q.shape[1])


def _fill_keys_from_layout(base: np.ndarray, noise: np.ndarray, src: np.ndarray,
                           sigma: float) -> np.ndarray:
    keys = base.copy()
    rep = src >= 0
    keys[..., rep, :] = base[..., src[rep], :] + sigma * noise[..., rep, :]
    return keys


def tiny_head_case(seed: int = 0, n: int = 96, budget: int = 64, window: int = 8,
                   gqa: int = 4, lam: float = 0.1, dup_frac: float = 0.30,
                   dup_sigma: float = 0.01, d: int = HEAD_DIM) -> DenseCase:
    """Single fp32 head with planted near-duplicates (the tiny workload)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keys = rng.standard_normal((n, d))
    pos, srcs = plant_near_duplicates(rng, keys, dup_frac, dup_sigma)
    values = rng.standard_normal((n, d))
    q = rng.standard_normal((gqa, window, d))
    return DenseCase(K=keys.astype(np.float32)[None], V=values.astype(np.float32)[None],
                     Q=q.astype(np.float32)[None], budget=budget, window=window, lam=lam,
                     dtype="f32", meta=dict(dup_positions=pos, dup_sources=srcs))


def dense_case_host(seed: int, batch: int, layers: int, kv_heads: int, gqa: int, n: int,
                    budget: int, window: int, lam: float, dtype: str = "bf16",
                    coverage: float = 0.40, sigma: float = 0.02, d: int = HEAD_DIM,
                    key_scale: float = 1.0) -> DenseCase:
    """Repeated-segment keys for batch*layers*kv_heads heads, drawn on the host.

    Heads are ordered (seq, layer, kv_head). One run layout per sequence is
    shared by all of its layers and heads (a restated span of text repeats in
    every head); fresh keys, noise, values and queries are per head.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    hps = layers * kv_heads
    bh = batch * hps
    layouts = np.stack([segment_layout(rng, n, coverage) for _ in range(batch)])
    K = np.empty((bh, n, d), np.float32)
    for b in range(batch):
        base = rng.standard_normal((hps, n, d)).astype(np.float32)
        noise = rng.standard_normal((hps, n, d)).astype(np.float32)
        K[b * hps:(b + 1) * hps] = key_scale * _fill_keys_from_layout(base, noise,
                                                                       layouts[b], sigma)
    V = rng.standard_normal((bh, n, d)).astype(np.float32)
    Q = rng.standard_normal((bh, gqa, window, d)).astype(np.float32)
    if dtype == "bf16":
        K, V, Q = bf16_round(K), bf16_round(V), bf16_round(Q)
    cov = float((layouts >= 0).mean())
    return DenseCase(K=K, V=V, Q=Q, budget=budget, window=window, lam=lam, dtype=dtype,
                     layouts=layouts, heads_per_seq=hps, meta=dict(coverage=cov))


def _torch_dtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def dense_case_device(seed: int, batch: int, layers: int, kv_heads: int, gqa: int, n: int,
                      budget: int, window: int, lam: float, dtype: str = "bf16",
                      coverage: float = 0.40, sigma: float = 0.02, d: int = HEAD_DIM,
                      device: str = "cuda", chunk: int = 512,
                      capacity: Optional[int] = None) -> DenseCase:
    """Same recipe as :func:`dense_case_host`, drawn with torch on the device.

    For workloads of thousands of heads (gigabytes of cache). Each chunk of
    heads has its own generator seed, so a head's values depend only on
    (seed, head). ``capacity`` >= n gives each head room for that many rows
    (the cache buffer of a decode loop); rows n..capacity-1 are zero.
    """
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    hps = layers * kv_heads
    bh = batch * hps
    cap = n if capacity is None else capacity
    layouts = np.stack([segment_layout(rng, n, coverage) for _ in range(batch)])
    tdt = _torch_dtype(dtype)
    K = torch.zeros((bh, cap, d), dtype=tdt, device=device)
    V = torch.zeros((bh, cap, d), dtype=tdt, device=device)
    Q = torch.empty((bh, gqa, window, d), dtype=tdt, device=device)
    seq_of_head = np.arange(bh) // hps
    lay_dev = torch.as_tensor(layouts, device=device)
    g = torch.Generator(device=device)
    for c0 in range(0, bh, chunk):
        c1 = min(bh, c0 + chunk)
        g.manual_seed(seed * 1_000_003 + c0)
        base = torch.randn((c1 - c0, n, d), generator=g, device=device)
        noise = torch.randn((c1 - c0, n, d), generator=g, device=device)
        src = lay_dev[torch.as_tensor(seq_of_head[c0:c1], device=device)]   # [c, n]
        rep = src >= 0
        idx = torch.where(rep, src, torch.arange(n, device=device)[None, :])
        copied = torch.gather(base, 1, idx[..., None].expand(-1, -1, d)) + sigma * noise
        keys = torch.where(rep[..., None], copied, base)
        K[c0:c1, :n] = keys.to(tdt)
        V[c0:c1, :n] = torch.randn((c1 - c0, n, d), generator=g, device=device).to(tdt)
        Q[c0:c1] = torch.randn((c1 - c0, gqa, window, d), generator=g,
                               device=device).to(tdt)
        del base, noise, copied, keys
    cov = float((layouts >= 0).mean())
    return DenseCase(K=K, V=V, Q=Q, budget=budget, window=window, lam=lam, dtype=dtype,
                     layouts=layouts, heads_per_seq=hps, meta=dict(coverage=cov, capacity=cap))


@dataclasses.dataclass
class PagedCase:
    """Paged cache inputs.

    K_pages, V_pages: [P, H, page_size, d]; page_table: [S, max_pages] int32
    (-1 = no page); seq_len, budget: [S] int32; Q: [S, H, G, w, d];
    free_list: initial free page ids (int32).
    """
    K_pages: object
    V_pages: object
    page_table: np.ndarray
    seq_len: np.ndarray
    budget: np.ndarray
    Q: object
    free_list: np.ndarray
    window: int
    lam: float
    page_size: int
    dtype: str
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def kv_heads(self) -> int:
        return int(self.K_pages.shape[1])


def _paged_layout(rng, seq_len, budget_frac, window, page_size, spare_pages, max_pages=None):
    s = len(seq_len)
    pages_per_seq = (seq_len + page_size - 1) // page_size
    maxp = int(pages_per_seq.max()) if max_pages is None else max_pages
    min_budget = page_size * int(math.ceil((window + 1) / page_size))
    budget = np.maximum(page_size * np.round(budget_frac * seq_len / page_size).astype(np.int64),
                        min_budget).astype(np.int32)
    total = int(pages_per_seq.sum())
    pool = total + spare_pages
    perm = rng.permutation(pool).astype(np.int32)
    table = np.full((s, maxp), -1, dtype=np.int32)
    off = 0
    for i in range(s):
        table[i, :pages_per_seq[i]] = perm[off:off + pages_per_seq[i]]
        off += int(pages_per_seq[i])
    free = perm[off:].copy()
    return table, budget, free, pool


def paged_case_host(seed: int, seq_len, budget_frac, kv_heads: int = 2, gqa: int = 2,
                    window: int = 8, lam: float = 0.1, dtype: str = "bf16",
                    coverage: float = 0.40, sigma: float = 0.02, page_size: int = PAGE_SIZE,
                    spare_pages: int = 8, d: int = HEAD_DIM) -> PagedCase:
    """Small paged cache drawn on the host, for tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_len = np.asarray(seq_len, dtype=np.int32)
    budget_frac = np.broadcast_to(np.asarray(budget_frac, dtype=np.float64), seq_len.shape)
    table, budget, free, pool = _paged_layout(rng, seq_len, budget_frac, window, page_size,
                                              spare_pages)
    Kp = rng.standard_normal((pool, kv_heads, page_size, d)).astype(np.float32)
    Vp = rng.standard_normal((pool, kv_heads, page_size, d)).astype(np.float32)
    for s, n in enumerate(seq_len):
        src = segment_layout(rng, int(n), coverage)
        base = rng.standard_normal((kv_heads, int(n), d)).astype(np.float32)
        noise = rng.standard_normal((kv_heads, int(n), d)).astype(np.float32)
        keys = _fill_keys_from_layout(base, noise, src, sigma)
        for t in range(int(n)):
            Kp[table[s, t // page_size], :, t % page_size] = keys[:, t]
    Q = rng.standard_normal((len(seq_len), kv_heads, gqa, window, d)).astype(np.float32)
    if dtype == "bf16":
        Kp, Vp, Q = bf16_round(Kp), bf16_round(Vp), bf16_round(Q)
    return PagedCase(K_pages=Kp, V_pages=Vp, page_table=table, seq_len=seq_len, budget=budget,
                     Q=Q, free_list=free, window=window, lam=lam, page_size=page_size,
                     dtype=dtype, meta=dict(pool=pool))


def paged_case_device(seed: int, seqs: int = 128, kv_heads: int = 8, gqa: int = 4,
                      n_min: int = 2048, n_max: int = 32768, frac_min: float = 0.10,
                      frac_max: float = 0.34, window: int = 8, lam: float = 0.1,
                      dtype: str = "bf16", coverage: float = 0.40, sigma: float = 0.02,
                      page_size: int = PAGE_SIZE, spare_pages: int = 1024,
                      d: int = HEAD_DIM, device: str = "cuda") -> PagedCase:
    """The paged ragged workload drawn with torch on the device.

    Lengths U{n_min..n_max}, budget fraction U[frac_min, frac_max] rounded to a
    page (at least one page past the window), 16-token pages, a seeded
    permutation of the pool assigning physical pages to (seq, logical page) in
    order, and the spare pages as the initial free list.
    """
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_len = rng.integers(n_min, n_max + 1, size=seqs).astype(np.int32)
    frac = rng.uniform(frac_min, frac_max, size=seqs)
    table, budget, free, pool = _paged_layout(rng, seq_len, frac, window, page_size,
                                              spare_pages)
    tdt = _torch_dtype(dtype)
    Kp = torch.zeros((pool, kv_heads, page_size, d), dtype=tdt, device=device)
    Vp = torch.zeros((pool, kv_heads, page_size, d), dtype=tdt, device=device)
    g = torch.Generator(device=device)
    for s in range(seqs):
        n = int(seq_len[s])
        npg = (n + page_size - 1) // page_size
        src = segment_layout(rng, n, coverage)
        g.manual_seed(seed * 1_000_003 + s)
        base = torch.randn((kv_heads, npg * page_size, d), generator=g, device=device)
        noise = torch.randn((kv_heads, n, d), generator=g, device=device)
        src_t = torch.as_tensor(src, device=device)
        rep = src_t >= 0
        idx = torch.where(rep, src_t, torch.arange(n, device=device))
        keys = base.clone()
        keys[:, :n] = torch.where(rep[None, :, None], base[:, idx] + sigma * noise, base[:, :n])
        vals = torch.randn((kv_heads, npg * page_size, d), generator=g, device=device)
        pages = torch.as_tensor(table[s, :npg].astype(np.int64), device=device)
        Kp[pages] = keys.view(kv_heads, npg, page_size, d).permute(1, 0, 2, 3).to(tdt)
        Vp[pages] = vals.view(kv_heads, npg, page_size, d).permute(1, 0, 2, 3).to(tdt)
        del base, noise, keys, vals
    g.manual_seed(seed * 1_000_003 + seqs)
    Q = torch.randn((seqs, kv_heads, gqa, window, d), generator=g, device=device).to(tdt)
    return PagedCase(K_pages=Kp, V_pages=Vp, page_table=table, seq_len=seq_len, budget=budget,
                     Q=Q, free_list=free, window=window, lam=lam, page_size=page_size,
                     dtype=dtype, meta=dict(pool=pool))
