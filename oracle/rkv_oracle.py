"""Plain float64 CPU oracle for the R-KV decode-time compression step.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` are the only code that may import
this module. The library (``decode_kv_cache_03_amd``) never calls it, and the
two share no code: this file is written from the pages, not from the kernels.

Pages cited (by title; sections in quotes):
  [P1] "R-KV: decoding-time KV cache compression for reasoning models"
       (hysenlabs project page)
  [P2] sourcepulse project summary of R-KV (its "How It Works" section)
  [P3] "R-KV: Redundancy-aware KV Cache Compression for Reasoning Models"
       (atlas.scime.ai AI-extracted paper summary)

What the method computes, per (layer, KV head) over the N buffered candidates:
  * importance I from attention weights [P2 "How It Works"; P3 "Approach"],
    pooled over the query heads of a GQA group by max, mean pooling being the
    worse ablation [P3 "Measured effects reported in the paper", last row];
  * redundancy R from the cosine similarity of key vectors, to find and prune
    near-duplicates [P2 "How It Works"; P3 "Approach"; P1 "How this differs
    from attention-sink and heavy-hitter eviction"];
  * the joint score Z = lam*I - (1-lam)*R [P3 "Approach"];
  * a recent window exempt from eviction [P1 "What the redundancy scoring
    actually does at decode time"], and the top tokens by Z kept within the
    budget [P2 "How It Works"];
  * physical eviction: the kept rows are compacted and freed cache blocks go
    back to the allocator [P1 "What the redundancy scoring actually does at
    decode time"; "How this differs ..."].

Readings taken where the pages leave a step open (each is also listed with its
reasoning in the design notes of the repository):
  R1  R_i = max over EARLIER candidates j < i of cos(k_i, k_j); R_0 = 0. P1
      describes the score as similarity to what is already retained and the
      eviction as removing the duplicate, i.e. the later copy.
  R2  A zero-norm key has cosine 0 with every key.
  R3  Importance uses the last w decode queries of each of the G query heads
      of the group; query r of the window (r = 0..w-1) sees keys j <= N-w+r.
  R4  Logits are q.k / sqrt(d); softmax over the visible keys; mean over the w
      queries of a head, then max over the G heads.
  R5  No rescaling of I or R: Z is taken literally.
  R6  The window (last w candidates) is always kept; the other B-w slots go to
      the candidates with the largest Z, ties to the smaller index; kept
      indices are returned ascending; -0.0 and +0.0 are equal.
  R7  N <= B keeps everything; B <= w is invalid.
  R8  Paged mode: each (sequence, head) compacts its kept rows into logical
      slots 0..B_s-1 of its own sequence; pages p >= B_s/page_size of the
      sequence are freed in (sequence, page) ascending order and their page
      table entries become -1.

Variants of those readings, selected by keyword arguments (defaults = R1-R8):
  symmetric=True   R_i = max over every other candidate j != i of
                   cos(k_i, k_j): the plain symmetric reading of R1, which
                   scores both copies of a duplicate as redundant.
  causal=False     every window query sees all N candidates (R3 without the
                   in-window causal mask).
  pool="mean"      I_j = mean over the G query heads of the per-head window
                   mean (the ablation that replaces max pooling of GQA
                   attention scores [P3 "Measured effects reported in the
                   paper", last row]).
  Head-shared selection (compress_shared): the heads that must evict one
  token set, as the tensor-parallel ranks of a layer do after their
  eviction-score all-reduce [P1 "What the redundancy scoring actually does
  at decode time"], select on the SUM of their Z (an all-reduce's default
  reduction); the window and the top B-w of that sum are kept by every head.
  On pages (compress_paged(shared_heads=True)) the group is a sequence's H
  heads: one token set per sequence, the layout vLLM's token-major pages
  need.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def key_norms(K) -> np.ndarray:
    """Euclidean norm of every key row, K [N, d] -> [N]."""
    K = _f64(K)
    return np.sqrt(np.sum(K * K, axis=1))


def attention_probs(K, Q, window: int, causal: bool = True) -> np.ndarray:
    """Softmax attention of the window queries over the N candidates (reading R3, R4).

    K [N, d]; Q [G, w, d] -> P [G, w, N], each row summing to 1 over the keys
    it can see and 0 on the keys it cannot. causal=False lets every window
    query see all N keys.
    """
    K = _f64(K)
    Q = _f64(Q)
    n, d = K.shape
    g, w, _ = Q.shape
    assert w == window
    logits = (Q.reshape(g * w, d) @ K.T) / math.sqrt(d)          # [G*w, N]
    logits = logits.reshape(g, w, n)
    if causal:
        # Window query r attends to keys 0 .. N-w+r (causal inside the window).
        visible = np.arange(n)[None, :] <= (n - w + np.arange(w))[:, None]   # [w, N]
        logits = np.where(visible[None], logits, -np.inf)
    m = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=2, keepdims=True)


def importance(K, Q, window: int, causal: bool = True, pool: str = "max") -> np.ndarray:
    """I_j = max (or, pool="mean", mean) over query heads g of the mean over
    window queries r of P[g, r, j]."""
    per_head = attention_probs(K, Q, window, causal=causal).mean(axis=1)   # [G, N]
    if pool == "max":
        return per_head.max(axis=0)
    if pool == "mean":
        return per_head.mean(axis=0)
    raise ValueError(f"unknown pooling {pool!r}")


def _cosines(K, norms, i, cols) -> np.ndarray:
    """cos(k_i, k_j) for j in cols; 0 where a norm is 0 (reading R2)."""
    dots = K[cols] @ K[i]
    denom = norms[cols] * norms[i]
    return np.divide(dots, denom, out=np.zeros(len(cols)), where=denom > 0)


def _redundancy_of(K, norms, i: int, symmetric: bool) -> float:
    n = K.shape[0]
    if symmetric:
        cols = np.concatenate([np.arange(i), np.arange(i + 1, n)])
    else:
        cols = np.arange(i)
    if len(cols) == 0:
        return 0.0
    return float(_cosines(K, norms, i, cols).max())


def redundancy(K, symmetric: bool = False) -> np.ndarray:
    """R_i = max_{j<i} cos(k_i, k_j), R_0 = 0 (readings R1, R2); with
    symmetric=True, max over every j != i."""
    K = _f64(K)
    norms = key_norms(K)
    return np.array([_redundancy_of(K, norms, i, symmetric) for i in range(K.shape[0])])


def redundancy_rows(K, rows, symmetric: bool = False) -> np.ndarray:
    """R_i for the listed rows only (same definition as :func:`redundancy`)."""
    K = _f64(K)
    norms = key_norms(K)
    return np.array([_redundancy_of(K, norms, int(i), symmetric) for i in rows])


def joint_score(I, R, lam: float) -> np.ndarray:
    """Z = lam*I - (1-lam)*R."""
    return lam * _f64(I) - (1.0 - lam) * _f64(R)


def select(Z, n: int, budget: int, window: int) -> np.ndarray:
    """Kept candidate indices, ascending (readings R6, R7)."""
    if budget <= window:
        raise ValueError("budget must exceed window")
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    Z = _f64(Z)
    cand = n - window
    idx = np.arange(cand)
    # Primary key: Z descending; secondary key: index ascending.
    order = np.lexsort((idx, -Z[:cand]))
    chosen = order[:budget - window]
    return np.sort(np.concatenate([chosen, np.arange(cand, n)])).astype(np.int64)


def scores_head(K, Q, window: int, lam: float, symmetric: bool = False, causal: bool = True,
                pool: str = "max"):
    """(I, R, Z) of one head under the chosen readings."""
    I = importance(K, Q, window, causal=causal, pool=pool)
    R = redundancy(K, symmetric=symmetric)
    return I, R, joint_score(I, R, lam)


def compress_head(K, V, Q, budget: int, window: int, lam: float, symmetric: bool = False,
                  causal: bool = True, pool: str = "max") -> dict:
    """The whole step for one head: scores, selection and the compacted rows.

    K, V [N, d]; Q [G, w, d]. Returns dict(kept, K_out, V_out, I, R, Z), the
    scores being None when N <= budget (nothing is scored). The keyword
    arguments select the reading variants listed in the module header.
    """
    K = np.asarray(K)
    V = np.asarray(V)
    n = K.shape[0]
    if budget <= window:
        raise ValueError("budget must exceed window")
    if n <= budget:
        kept = np.arange(n, dtype=np.int64)
        return dict(kept=kept, K_out=K[kept].copy(), V_out=V[kept].copy(),
                    I=None, R=None, Z=None)
    if symmetric or not causal or pool != "max":
        I, R, Z = scores_head(K, Q, window, lam, symmetric=symmetric, causal=causal, pool=pool)
    else:
        I = importance(K, Q, window)
        R = redundancy(K)
        Z = joint_score(I, R, lam)
    kept = select(Z, n, budget, window)
    return dict(kept=kept, K_out=K[kept].copy(), V_out=V[kept].copy(), I=I, R=R, Z=Z)


def compress_dense(K, V, Q, budget: int, window: int, lam: float, heads=None, **variant) -> list:
    """:func:`compress_head` over heads (all, or the listed ones). K [Bh, N, d]."""
    heads = range(K.shape[0]) if heads is None else heads
    return [compress_head(K[h], V[h], Q[h], budget, window, lam, **variant) for h in heads]


def compress_shared(K, V, Q, budget: int, window: int, lam: float, **variant) -> dict:
    """Head-shared selection over the H heads of one group (see the module
    header): K, V [H, N, d]; Q [H, G, w, d]. Each head's Z is computed as in
    :func:`compress_head`; the group selects once on Z_sum = sum over heads
    of Z; every head keeps those indices. Returns dict(kept, K_out [H, B, d],
    V_out, Z [H, N], Z_sum), scores None when N <= budget."""
    K = np.asarray(K)
    V = np.asarray(V)
    H, n = K.shape[0], K.shape[1]
    if budget <= window:
        raise ValueError("budget must exceed window")
    if n <= budget:
        kept = np.arange(n, dtype=np.int64)
        return dict(kept=kept, K_out=K[:, kept].copy(), V_out=V[:, kept].copy(), Z=None,
                    Z_sum=None)
    Z = np.stack([scores_head(K[h], Q[h], window, lam, **variant)[2] for h in range(H)])
    Z_sum = Z.sum(axis=0)
    kept = select(Z_sum, n, budget, window)
    return dict(kept=kept, K_out=K[:, kept].copy(), V_out=V[:, kept].copy(), Z=Z, Z_sum=Z_sum)


def logical_rows(pages, page_table_row, n: int, head: int, page_size: int) -> np.ndarray:
    """Rows 0..n-1 of one (sequence, head) read through its page table row."""
    t = np.arange(n)
    return np.asarray(pages)[page_table_row[t // page_size], head, t % page_size]


def return_pages(page_table, seq_len, budget, free_list, page_size: int):
    """Block return after compaction (reading R8) [P1 "What the redundancy
    scoring actually does at decode time": freed blocks go back to the
    allocator].

    A compressed sequence (N_s > B_s) keeps B_s tokens in its first
    B_s/page_size pages; each later page it held (up to ceil(N_s/page_size))
    is appended to the free list, sequences in order and pages in order within
    a sequence, and its table entry becomes -1. Returns (new table, new free
    list); the inputs are not modified.
    """
    table = np.array(page_table, copy=True)
    freed = [int(x) for x in free_list]
    for s in range(table.shape[0]):
        n = int(seq_len[s])
        b = int(budget[s])
        if n <= b:
            continue
        held = (n + page_size - 1) // page_size
        for p in range(b // page_size, held):
            freed.append(int(table[s, p]))
            table[s, p] = -1
    return table, np.asarray(freed, dtype=np.int64)


def compress_paged(K_pages, V_pages, page_table, seq_len, budget, Q, free_list,
                   window: int, lam: float, page_size: int, shared_heads: bool = False,
                   **variant) -> dict:
    """Paged compression with page return (reading R8).

    K_pages, V_pages [P, H, page_size, d]; page_table [S, maxp]; seq_len,
    budget [S]; Q [S, H, G, w, d]; free_list: the free page ids before the
    call. Returns dict(K_pages, V_pages, page_table, free_list, kept) where
    kept[s][h] are the kept logical indices and the pages are new arrays.
    The keyword arguments select the reading variants, as in compress_head.
    shared_heads: the H heads of each sequence select together, as in
    compress_shared (one token set per sequence, chosen on the sum of the
    heads' Z); the pages and the page return are handled as before.
    """
    Kp = np.array(K_pages, copy=True)
    Vp = np.array(V_pages, copy=True)
    kept_all = []
    n_seq, heads = np.shape(page_table)[0], Kp.shape[1]
    for s in range(n_seq):
        n = int(seq_len[s])
        b = int(budget[s])
        if b % page_size != 0:
            raise ValueError("paged budget must be a multiple of the page size")
        Kl = [logical_rows(K_pages, page_table[s], n, h, page_size) for h in range(heads)]
        Vl = [logical_rows(V_pages, page_table[s], n, h, page_size) for h in range(heads)]
        if shared_heads:
            res = compress_shared(np.stack(Kl), np.stack(Vl), np.asarray(Q)[s], b, window, lam,
                                  **variant)
            kept_s = [res["kept"]] * heads
        else:
            kept_s = [compress_head(Kl[h], Vl[h], np.asarray(Q)[s, h], b, window, lam,
                                    **variant)["kept"] for h in range(heads)]
        if n > b:
            for h in range(heads):
                kept = kept_s[h]
                r = np.arange(len(kept))
                Kp[page_table[s][r // page_size], h, r % page_size] = Kl[h][kept]
                Vp[page_table[s][r // page_size], h, r % page_size] = Vl[h][kept]
        kept_all.append(kept_s)
    table, freed = return_pages(page_table, seq_len, budget, free_list, page_size)
    return dict(K_pages=Kp, V_pages=Vp, page_table=table, free_list=freed, kept=kept_all)
