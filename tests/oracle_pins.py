"""Pins for the CPU oracle: checks against facts fixed by the pages and by mathematics.

Each ``check_*`` raises AssertionError on failure. ``test_oracle_pins.py`` runs
them on the oracle as written; ``test_oracle_mutants.py`` plants plausible
mistakes in the oracle and confirms at least one check fails for each.

Pinned facts and where they come from:
  * pure-Python brute force (independent loops, exhaustive subset search) on
    tiny heads agrees with the oracle;
  * lam = 1 reduces Z to the importance alone and the selection to an
    attention top-k (the pages' attention-only ablation, SnapKV-like);
    lam = 0 reduces Z to -R (the redundancy-only ablation);
  * an exact copy (up to a positive scale) of an earlier key has cosine 1,
    the largest redundancy possible; orthogonal keys have redundancy 0;
    cosine is invariant to scaling keys;
  * zero (or key-orthogonal) queries give a uniform causal softmax, whose
    pooled importance has a closed form;
  * softmax rows sum to one; pooled importance is at most G in total;
    identical query heads pool to the single-head importance;
  * a hand-worked 2-D example with keys at known angles;
  * structure: output size, window kept, ascending order, K'/V' = gather;
  * paged page return, by invariants that do not restate the oracle's loop:
    the live table entries and the free list are an exact partition of the
    pool before and after; the free list only grows at its end, by the pages
    a sequence no longer needs (ceil(N_s/ps) - ceil(min(N_s, B_s)/ps) each);
    the pages a sequence keeps are its first ones, unchanged; the freed ids,
    located in the old table, ascend by (sequence, page);
  * paged data: live slots hold the kept rows; nothing else changes;
  * redundancy of listed rows: equal to the brute force's R at those rows,
    to 1 at planted exact copies and to 0 for orthogonal keys.

Pins of the reading variants (symmetric redundancy, importance without the
in-window causal mask, mean pooling over the GQA heads) and of head-shared
selection:
  * the brute force, which implements each variant by its own loops, agrees;
  * symmetric: the 2-D example's values follow from the angles; both copies
    of a planted duplicate reach 1; orthogonal keys give 0;
  * unmasked: zero queries give exactly 1/N for every key; every softmax row
    covers all N keys;
  * pooling: with orthogonal unit keys, queries built from logarithms give
    softmax rows equal to chosen distributions, so max and mean pooling have
    closed forms;
  * shared selection: exhaustive search over subsets of the summed scores;
    heads that are copies of one head select what that head selects alone.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import bruteforce as bf
from oracle import rkv_oracle as orc


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def tiny_case(seed):
    rng = _rng(seed)
    n = int(rng.integers(6, 12))
    d = int(rng.integers(2, 9))
    g = int(rng.integers(1, 4))
    w = int(rng.integers(1, 4))
    b = int(rng.integers(w + 1, n))
    lam = float(rng.choice([0.1, 0.3, 0.7, 0.9]))
    K = rng.standard_normal((n, d))
    # a near-duplicate and an exact copy make redundancy non-trivial
    K[n - 2] = K[1] + 0.01 * rng.standard_normal(d)
    K[n // 2] = 2.0 * K[0]
    V = rng.standard_normal((n, d))
    Q = rng.standard_normal((g, w, d))
    return K, V, Q, b, w, lam


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b) / np.maximum(1.0, np.abs(b))
    assert np.all(err <= tol), f"max rel err {err.max()}"


def check_bruteforce(seed):
    K, V, Q, b, w, lam = tiny_case(seed)
    o = orc.compress_head(K, V, Q, b, w, lam)
    r = bf.compress_head_bf(K.tolist(), V.tolist(), Q.tolist(), b, w, lam)
    _close(o["I"], r["I"])
    _close(o["R"], r["R"])
    _close(o["Z"], r["Z"])
    assert list(o["kept"]) == list(r["kept"]), (list(o["kept"]), r["kept"])


def check_select_ties(seed):
    """Integer-valued Z with many exact ties, window scored lowest."""
    rng = _rng(seed)
    n = int(rng.integers(7, 13))
    w = int(rng.integers(1, 4))
    b = int(rng.integers(w + 1, n))
    Z = rng.integers(-2, 3, size=n).astype(np.float64)
    Z[n - w:] = -100.0
    if seed % 2:
        Z[rng.integers(0, n - w)] = -0.0
    kept = orc.select(Z, n, b, w)
    assert list(kept) == bf.select_bf(Z.tolist(), n, b, w)


def check_lambda_one(seed):
    K, V, Q, b, w, _ = tiny_case(seed)
    n = K.shape[0]
    o = orc.compress_head(K, V, Q, b, w, 1.0)
    assert np.array_equal(o["Z"], o["I"])
    I = orc.importance(K, Q, w)
    top = np.argsort(-I[:n - w], kind="stable")[:b - w]
    assert list(o["kept"]) == sorted(list(top) + list(range(n - w, n)))


def check_lambda_zero(seed):
    K, V, Q, b, w, _ = tiny_case(seed)
    n = K.shape[0]
    o = orc.compress_head(K, V, Q, b, w, 0.0)
    assert np.array_equal(o["Z"], -o["R"])
    R = orc.redundancy(K)
    least = np.argsort(R[:n - w], kind="stable")[:b - w]
    assert list(o["kept"]) == sorted(list(least) + list(range(n - w, n)))


def check_duplicates(seed):
    rng = _rng(seed)
    n, d, w = 40, 16, 4
    b = 30
    K = rng.standard_normal((n, d))
    copies = []
    for t in range(5, n - w, 3):          # 11 later copies outside the window
        src = int(rng.integers(0, t))
        K[t] = float(rng.choice([0.5, 1.0, 3.0])) * K[src]
        copies.append(t)
    assert len(copies) >= n - b
    R = orc.redundancy(K)
    for t in copies:
        assert abs(R[t] - 1.0) <= 1e-12, R[t]
        assert R[t] >= R.max() - 1e-12
    Q = rng.standard_normal((2, w, d))
    kept = orc.compress_head(K, K, Q, b, w, 0.0)["kept"]
    evicted = sorted(set(range(n)) - set(kept.tolist()))
    assert set(evicted) <= set(copies), (evicted, copies)


def check_orthogonal(seed):
    rng = _rng(seed)
    d = 16
    n = int(rng.integers(4, d + 1))
    basis = np.eye(d)[rng.permutation(d)[:n]] * rng.uniform(0.5, 3.0, size=(n, 1))
    R = orc.redundancy(basis)
    assert np.array_equal(R, np.zeros(n))
    Q = rng.standard_normal((2, 2, d))
    o = orc.compress_head(basis, basis, Q, max(3, n - 2), 2, 0.3) if n > 3 else None
    if o is not None and o["Z"] is not None:
        _close(o["Z"], 0.3 * o["I"], 1e-15)


def check_scale_invariance(seed):
    rng = _rng(seed)
    K = rng.standard_normal((30, 12))
    K[20] = K[3]
    R = orc.redundancy(K)
    for s in (0.25, 4.0, 1024.0):
        _close(orc.redundancy(K * s), R, 1e-12)


def uniform_importance(n, w):
    """Closed form of the pooled importance when every logit is equal."""
    out = np.zeros(n)
    for j in range(n):
        # window query r sees keys 0 .. n-w+r, i.e. n-w+r+1 keys
        out[j] = sum(1.0 / (n - w + r + 1) for r in range(w) if j <= n - w + r) / w
    return out


def check_zero_queries(seed):
    rng = _rng(seed)
    n = int(rng.integers(5, 60))
    w = int(rng.integers(1, min(8, n)))
    g = int(rng.integers(1, 5))
    d = 8
    K = rng.standard_normal((n, d))
    I = orc.importance(K, np.zeros((g, w, d)), w)
    _close(I, uniform_importance(n, w), 1e-13)
    # queries orthogonal to every key give the same uniform softmax
    K2 = np.concatenate([rng.standard_normal((n, d - 1)), np.zeros((n, 1))], axis=1)
    Qo = np.zeros((g, w, d))
    Qo[..., -1] = rng.standard_normal((g, w))
    _close(orc.importance(K2, Qo, w), uniform_importance(n, w), 1e-13)
    # one zero head beside a random head: max pooling never drops below the
    # uniform head, and equals the larger of the two heads' window means
    Qm = np.concatenate([np.zeros((1, w, d)), 3.0 * rng.standard_normal((1, w, d))])
    Im = orc.importance(K, Qm, w)
    P1 = orc.attention_probs(K, Qm[1:], w)[0].mean(axis=0)
    _close(Im, np.maximum(uniform_importance(n, w), P1), 1e-13)


def check_logit_scale(seed):
    """One window query, one key aligned with it: softmax of a single logit
    a = q.k/sqrt(d) among N-1 zero logits is e^a / (e^a + N - 1)."""
    rng = _rng(seed)
    d = int(rng.choice([4, 16, 64]))
    n = int(rng.integers(3, 20))
    K = np.zeros((n, d))
    K[:, 1:] = rng.standard_normal((n, d - 1))
    K[0, 0] = 2.0
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 3.0                       # q.k_0 = 6, q.k_j = 0 for j > 0
    a = 6.0 / math.sqrt(d)
    I = orc.importance(K, q, 1)
    _close(I[0], math.exp(a) / (math.exp(a) + n - 1), 1e-14)


def check_softmax_rows(seed):
    rng = _rng(seed)
    n, d, g, w = 50, 16, 3, 5
    K = rng.standard_normal((n, d))
    Q = 2.0 * rng.standard_normal((g, w, d))
    P = orc.attention_probs(K, Q, w)
    _close(P.sum(axis=2), np.ones((g, w)), 1e-13)
    for r in range(w):
        assert np.all(P[:, r, n - w + r + 1:] == 0.0)
        assert np.all(P[:, r, :n - w + r + 1] > 0.0)
    I = orc.importance(K, Q, w)
    assert I.sum() <= g + 1e-12
    assert np.all(I >= P.mean(axis=1).min(axis=0) - 1e-15)


def check_identical_heads(seed):
    rng = _rng(seed)
    n, d, w = 30, 8, 4
    K = rng.standard_normal((n, d))
    q = rng.standard_normal((1, w, d))
    _close(orc.importance(K, np.repeat(q, 4, axis=0), w), orc.importance(K, q, w), 1e-15)


def check_hand_example(seed=0):
    """2-D keys at known angles; zero queries; lam = 0 and lam = 1."""
    K = np.array([[1.0, 0.0], [0.0, 2.0], [3.0, 3.0], [-1.0, 0.0], [2.0, 0.0], [0.0, -1.0]])
    R = orc.redundancy(K)
    # k1 is orthogonal to k0; k2 is at 45 degrees to both; k3 is opposite k0,
    # orthogonal to k1, 135 degrees from k2; k4 is parallel to k0; k5 is
    # orthogonal to k0, k3, k4 and opposite k1.
    expect = [0.0, 0.0, math.sqrt(0.5), 0.0, 1.0, 0.0]
    _close(R, expect, 1e-15)
    Q = np.zeros((1, 1, 2))
    I = orc.importance(K, Q, 1)
    _close(I, np.full(6, 1.0 / 6.0), 1e-15)
    # lam = 0: Z = -R = [0, 0, -.707, 0, -1, 0]; window {5}; three of 0..4 by Z
    assert list(orc.compress_head(K, K, Q, 4, 1, 0.0)["kept"]) == [0, 1, 3, 5]
    # lam = 1 with uniform I: all ties, the earliest indices win
    assert list(orc.compress_head(K, K, Q, 4, 1, 1.0)["kept"]) == [0, 1, 2, 5]
    # lam = 0.5: Z = (1/6 - R)/2 -> 4 lowest, then 2; keep 0, 1, 3
    assert list(orc.compress_head(K, K, Q, 4, 1, 0.5)["kept"]) == [0, 1, 3, 5]


def check_structure(seed):
    rng = _rng(seed)
    n = int(rng.integers(10, 80))
    w = int(rng.integers(1, 6))
    b = int(rng.integers(w + 1, n + 10))
    d = 8
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    Q = rng.standard_normal((2, w, d))
    o = orc.compress_head(K, V, Q, b, w, 0.1)
    kept = o["kept"]
    assert len(kept) == min(n, b)
    assert np.all(np.diff(kept) > 0)
    if n > b:
        assert set(range(n - w, n)) <= set(kept.tolist())
    assert np.array_equal(o["K_out"], K[kept])
    assert np.array_equal(o["V_out"], V[kept])


def check_page_return(table0, free0, table1, free1, seq_len, budget, ps, pool):
    """Invariants of the page return, stated without its loop.

    table0/free0: state before (live entries of the table plus the free list
    must be an exact partition of the pool's page ids 0..pool-1); table1/free1:
    after. A sequence of L tokens occupies ceil(L/ps) pages; after the call a
    sequence holds min(N_s, B_s) tokens."""
    table0 = np.asarray(table0)
    table1 = np.asarray(table1)
    free0 = [int(x) for x in free0]
    free1 = [int(x) for x in free1]
    S = len(seq_len)
    held0 = [-(-int(n) // ps) for n in seq_len]
    held1 = [-(-min(int(n), int(b)) // ps) for n, b in zip(seq_len, budget)]

    def live(t):
        return [int(x) for s in range(S) for x in t[s] if x >= 0]

    assert sorted(live(table0) + free0) == list(range(pool)), "initial state is not a partition"
    # the free list keeps its entries and grows at the end by the pages given up
    assert free1[:len(free0)] == free0, "existing free-list entries changed"
    assert len(free1) - len(free0) == sum(h0 - h1 for h0, h1 in zip(held0, held1)), \
        "wrong number of pages returned"
    # every page is either live in the table or free, exactly once
    assert sorted(live(table1) + free1) == list(range(pool)), "pool not conserved"
    for s in range(S):
        # the pages kept are the sequence's first ones, unchanged; the ones
        # after them no longer belong to it; the columns past its old length
        # are untouched
        assert np.array_equal(table1[s, :held1[s]], table0[s, :held1[s]]), f"seq {s}: kept pages moved"
        assert np.all(table1[s, held1[s]:held0[s]] < 0), f"seq {s}: a returned page is still mapped"
        assert np.array_equal(table1[s, held0[s]:], table0[s, held0[s]:]), f"seq {s}: columns past N_s"
    # the freed ids, found in the old table, ascend by (sequence, page)
    where = {int(table0[s, p]): (s, p) for s in range(S) for p in range(held0[s])}
    at = [where[x] for x in free1[len(free0):]]
    assert at == sorted(at), "freed pages out of (sequence, page) order"


def check_paged(seed):
    from synth import paged_case_host
    ps = 16
    lens = [40, 100, 16, 130, 33]
    fracs = [0.5, 0.3, 0.9, 0.4, 0.9]
    case = paged_case_host(seed, lens, fracs, kv_heads=2, gqa=2, window=4, lam=0.1,
                           dtype="f32", page_size=ps, spare_pages=5, d=8)
    out = orc.compress_paged(case.K_pages, case.V_pages, case.page_table, case.seq_len,
                             case.budget, case.Q, case.free_list, case.window, case.lam, ps)
    check_page_return(case.page_table, case.free_list, out["page_table"], out["free_list"],
                      case.seq_len, case.budget, ps, case.meta["pool"])
    # the page return step alone, on random lengths and budgets (pages of 1,
    # 4 and 16 tokens; some sequences compressed, some not)
    rng = _rng(seed)
    for ps_r in (1, 4, 16):
        S = int(rng.integers(2, 7))
        n = rng.integers(1, 12 * ps_r, size=S)
        b = ps_r * rng.integers(1, 8, size=S)
        held = -(-n // ps_r)
        maxp = int(held.max()) + int(rng.integers(0, 3))
        pool = int(held.sum()) + int(rng.integers(0, 5))
        perm = rng.permutation(pool)
        table = np.full((S, maxp), -1, dtype=np.int64)
        off = 0
        for s in range(S):
            table[s, :held[s]] = perm[off:off + held[s]]
            off += int(held[s])
        free = perm[off:]
        t1, f1 = orc.return_pages(table, n, b, free, ps_r)
        check_page_return(table, free, t1, f1, n, b, ps_r, pool)
        assert np.array_equal(table, np.asarray(table)), "inputs modified"
    live = np.zeros(case.K_pages.shape[:1] + case.K_pages.shape[1:3], dtype=bool)
    for s, n in enumerate(case.seq_len):
        n = int(n)
        for h in range(case.kv_heads):
            kept = out["kept"][s][h]
            assert len(kept) == min(n, int(case.budget[s]))
            for r, src in enumerate(kept):
                pg_src = case.page_table[s, src // ps]
                pg_dst = case.page_table[s, r // ps]
                assert np.array_equal(out["K_pages"][pg_dst, h, r % ps],
                                      case.K_pages[pg_src, h, src % ps])
                assert np.array_equal(out["V_pages"][pg_dst, h, r % ps],
                                      case.V_pages[pg_src, h, src % ps])
                live[pg_dst, h, r % ps] = True
    assert np.array_equal(out["K_pages"][~live], case.K_pages[~live])
    assert np.array_equal(out["V_pages"][~live], case.V_pages[~live])


def check_redundancy_rows(seed):
    """R of listed rows: the brute force at those rows on tiny heads (both
    readings); 1 at planted exact copies and 0 for orthogonal keys on a larger
    head."""
    rng = _rng(seed)
    n = int(rng.integers(8, 30))
    d = int(rng.integers(2, 10))
    K = rng.standard_normal((n, d))
    K[n - 1] = 0.5 * K[2]
    K[n // 2] = K[1] + 0.01 * rng.standard_normal(d)
    rows = np.concatenate([[0, n - 1], rng.choice(n, size=5, replace=False)])
    for sym in (False, True):
        ref = bf.redundancy_bf(K.tolist(), symmetric=sym)
        _close(orc.redundancy_rows(K, rows, symmetric=sym), [ref[int(i)] for i in rows])
    n, d = 600, 64
    K = rng.standard_normal((n, d))
    copies = sorted(rng.choice(np.arange(100, n), size=20, replace=False).tolist())
    for t in copies:
        K[t] = float(rng.choice([0.25, 2.0])) * K[int(rng.integers(0, 100))]
    R = orc.redundancy_rows(K, copies + [0, 1, 50])
    _close(R[:len(copies)], np.ones(len(copies)), 1e-12)
    assert R[len(copies)] == 0.0 and R[len(copies) + 1] < 1.0 - 1e-6
    basis = np.eye(d)[rng.permutation(d)[:40]] * rng.uniform(0.5, 3.0, size=(40, 1))
    assert np.array_equal(orc.redundancy_rows(basis, np.arange(40)), np.zeros(40))


VARIANTS = [dict(symmetric=True), dict(causal=False), dict(pool="mean"),
            dict(symmetric=True, causal=False, pool="mean")]


def check_bruteforce_variants(seed):
    K, V, Q, b, w, lam = tiny_case(seed)
    for var in VARIANTS:
        o = orc.compress_head(K, V, Q, b, w, lam, **var)
        r = bf.compress_head_bf(K.tolist(), V.tolist(), Q.tolist(), b, w, lam, **var)
        _close(o["I"], r["I"])
        _close(o["R"], r["R"])
        _close(o["Z"], r["Z"])
        assert list(o["kept"]) == list(r["kept"]), (var, list(o["kept"]), r["kept"])


def check_symmetric_closed_forms(seed):
    # the 2-D keys of check_hand_example: each key's largest cosine to any
    # OTHER key, from the angles (k0 parallel to k4; k1 at 45 degrees to k2;
    # k2 at 45 degrees to k0, k1, k4; k3 orthogonal to k1 and k5, opposite or
    # obtuse to the rest; k5 orthogonal to k0, k3, k4)
    K = np.array([[1.0, 0.0], [0.0, 2.0], [3.0, 3.0], [-1.0, 0.0], [2.0, 0.0], [0.0, -1.0]])
    h = math.sqrt(0.5)
    _close(orc.redundancy(K, symmetric=True), [1.0, h, h, 0.0, 1.0, 0.0], 1e-15)
    # lam = 0: Z = -R_sym = [-1, -.71, -.71, 0, -1, 0]; window {5}; keep 3 of
    # 0..4: 3, then 1 and 2 (tied, both kept)
    Q = np.zeros((1, 1, 2))
    assert list(orc.compress_head(K, K, Q, 4, 1, 0.0, symmetric=True)["kept"]) == [1, 2, 3, 5]
    rng = _rng(seed)
    # planted duplicate pairs: source and copy both reach cosine 1
    n, d = 30, 16
    K = rng.standard_normal((n, d))
    pairs = [(2, 11), (5, 20), (7, 25)]
    for a, c in pairs:
        K[c] = float(rng.choice([0.5, 2.0])) * K[a]
    R = orc.redundancy(K, symmetric=True)
    for a, c in pairs:
        assert abs(R[a] - 1.0) <= 1e-12 and abs(R[c] - 1.0) <= 1e-12, (R[a], R[c])
    others = [i for i in range(n) if i not in {x for pr in pairs for x in pr}]
    assert R[others].max() < 1.0 - 1e-6
    # orthogonal keys: nothing is redundant under either reading
    basis = np.eye(d)[rng.permutation(d)[:10]] * rng.uniform(0.5, 3.0, size=(10, 1))
    assert np.array_equal(orc.redundancy(basis, symmetric=True), np.zeros(10))


def check_unmasked_closed_forms(seed):
    rng = _rng(seed)
    n = int(rng.integers(5, 60))
    w = int(rng.integers(1, min(8, n)))
    g = int(rng.integers(1, 5))
    d = 8
    K = rng.standard_normal((n, d))
    for pool in ("max", "mean"):
        I = orc.importance(K, np.zeros((g, w, d)), w, causal=False, pool=pool)
        _close(I, np.full(n, 1.0 / n), 1e-14)
    P = orc.attention_probs(K, 2.0 * rng.standard_normal((g, w, d)), w, causal=False)
    _close(P.sum(axis=2), np.ones((g, w)), 1e-13)
    assert np.all(P > 0.0)
    # a single key aligned with every window query: e^a / (e^a + N - 1) for
    # every query, so also for the window mean
    K = np.zeros((n, d))
    K[:, 1:] = rng.standard_normal((n, d - 1))
    K[0, 0] = 2.0
    q = np.zeros((1, w, d))
    q[0, :, 0] = 3.0
    a = 6.0 / math.sqrt(d)
    _close(orc.importance(K, q, w, causal=False)[0], math.exp(a) / (math.exp(a) + n - 1), 1e-14)


def check_pooling_closed_forms(seed):
    """Orthogonal unit keys e_pi(j) and queries whose pi(j)-th component is
    sqrt(d) * log(a_j): the logits are log a_j, so each softmax row is
    a / sum(a) exactly (up to exp/log rounding)."""
    rng = _rng(seed)
    d = 16
    n = int(rng.integers(4, d + 1))
    g = int(rng.integers(2, 5))
    perm = rng.permutation(d)[:n]
    K = np.eye(d)[perm]
    A = rng.uniform(0.1, 5.0, size=(g, n))
    Q = np.zeros((g, 1, d))
    Q[:, 0, perm] = math.sqrt(d) * np.log(A)
    P = A / A.sum(axis=1, keepdims=True)          # [g, n] per-head distributions
    _close(orc.importance(K, Q, 1), P.max(axis=0), 1e-13)
    _close(orc.importance(K, Q, 1, pool="mean"), P.mean(axis=0), 1e-13)
    # identical heads pool alike under either rule
    Qi = np.repeat(Q[:1], g, axis=0)
    _close(orc.importance(K, Qi, 1, pool="mean"), orc.importance(K, Qi, 1), 1e-15)


def check_shared(seed):
    rng = _rng(seed)
    H = int(rng.integers(2, 4))
    K0, V0, Q0, b, w, lam = tiny_case(seed)
    n, d = K0.shape
    Ks = rng.standard_normal((H, n, d))
    Ks[0] = K0
    Vs = rng.standard_normal((H, n, d))
    Qs = rng.standard_normal((H,) + Q0.shape)
    for var in (dict(), VARIANTS[seed % len(VARIANTS)]):
        o = orc.compress_shared(Ks, Vs, Qs, b, w, lam, **var)
        r = bf.compress_shared_bf(Ks.tolist(), Vs.tolist(), Qs.tolist(), b, w, lam, **var)
        assert list(o["kept"]) == r["kept"], (var, list(o["kept"]), r["kept"])
        for h in range(H):
            _close(o["Z"][h], r["Z"][h])
            assert np.array_equal(o["K_out"][h], Ks[h][o["kept"]])
            assert np.array_equal(o["V_out"][h], Vs[h][o["kept"]])
    # copies of one head (2 or 4: the sum of equal values is exact) select
    # what that head selects alone
    for copies in (2, 4):
        rep = lambda x: np.repeat(x[None], copies, axis=0)
        o = orc.compress_shared(rep(K0), rep(V0), rep(Q0), b, w, lam)
        assert list(o["kept"]) == list(orc.compress_head(K0, V0, Q0, b, w, lam)["kept"])


def check_paged_shared(seed):
    """Head-shared selection on pages: the page table and free list as for
    per-head selection (page return does not depend on which tokens are
    kept); every head of a compressed sequence keeps one set, the one the
    brute-force shared selection picks on the sequence's logical rows; the
    kept rows are moved exactly and nothing else changes. A pool whose heads
    are copies of one another selects what per-head selection selects."""
    from synth import paged_case_host
    ps = 4   # tiny sequences: the brute force enumerates every kept set
    lens, fracs = [10, 12, 7, 11], [0.6, 0.5, 0.9, 0.7]
    case = paged_case_host(seed, lens, fracs, kv_heads=3, gqa=2, window=2, lam=0.1,
                           dtype="f32", page_size=ps, spare_pages=3, d=4)
    var = VARIANTS[seed % len(VARIANTS)] if seed % 2 else dict()
    out = orc.compress_paged(case.K_pages, case.V_pages, case.page_table, case.seq_len,
                             case.budget, case.Q, case.free_list, case.window, case.lam, ps,
                             shared_heads=True, **var)
    check_page_return(case.page_table, case.free_list, out["page_table"], out["free_list"],
                      case.seq_len, case.budget, ps, case.meta["pool"])
    H = case.kv_heads
    live = np.zeros(case.K_pages.shape[:1] + case.K_pages.shape[1:3], dtype=bool)
    for s, n in enumerate(case.seq_len):
        n, b = int(n), int(case.budget[s])
        kept = [list(map(int, out["kept"][s][h])) for h in range(H)]
        assert all(k == kept[0] for k in kept), f"seq {s}: heads keep different sets"
        if n > b:
            Kl = [orc.logical_rows(case.K_pages, case.page_table[s], n, h, ps).tolist() for h in range(H)]
            Vl = [orc.logical_rows(case.V_pages, case.page_table[s], n, h, ps).tolist() for h in range(H)]
            r = bf.compress_shared_bf(Kl, Vl, np.asarray(case.Q)[s].tolist(), b, case.window,
                                      case.lam, **var)
            assert kept[0] == r["kept"], (s, kept[0], r["kept"])
        else:
            assert kept[0] == list(range(n))
        for h in range(H):
            for r_, src in enumerate(kept[h]):
                pg_src = case.page_table[s, src // ps]
                pg_dst = case.page_table[s, r_ // ps]
                assert np.array_equal(out["K_pages"][pg_dst, h, r_ % ps],
                                      case.K_pages[pg_src, h, src % ps])
                assert np.array_equal(out["V_pages"][pg_dst, h, r_ % ps],
                                      case.V_pages[pg_src, h, src % ps])
                live[pg_dst, h, r_ % ps] = True
    assert np.array_equal(out["K_pages"][~live], case.K_pages[~live])
    assert np.array_equal(out["V_pages"][~live], case.V_pages[~live])
    # heads that are copies of head 0 (2 or 4 of them: the sums are exact)
    for copies in (2, 4):
        Kc = np.repeat(case.K_pages[:, :1], copies, axis=1)
        Vc = np.repeat(case.V_pages[:, :1], copies, axis=1)
        Qc = np.repeat(np.asarray(case.Q)[:, :1], copies, axis=1)
        a = orc.compress_paged(Kc, Vc, case.page_table, case.seq_len, case.budget, Qc,
                               case.free_list, case.window, case.lam, ps, shared_heads=True)
        p = orc.compress_paged(Kc, Vc, case.page_table, case.seq_len, case.budget, Qc,
                               case.free_list, case.window, case.lam, ps)
        for s in range(len(lens)):
            for h in range(copies):
                assert list(a["kept"][s][h]) == list(p["kept"][s][h])
        assert np.array_equal(a["K_pages"], p["K_pages"]) and np.array_equal(a["V_pages"], p["V_pages"])


ALL_CHECKS = [check_bruteforce, check_select_ties, check_lambda_one, check_lambda_zero,
              check_duplicates, check_orthogonal, check_scale_invariance, check_zero_queries,
              check_softmax_rows, check_identical_heads, check_logit_scale, check_hand_example, check_structure,
              check_paged, check_bruteforce_variants, check_symmetric_closed_forms,
              check_unmasked_closed_forms, check_pooling_closed_forms, check_shared,
              check_redundancy_rows, check_paged_shared]
