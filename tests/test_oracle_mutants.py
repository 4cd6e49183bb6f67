"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each one.

Every mutant below is the oracle with one step changed: a dropped or swapped
pooling, a wrong mask or scale, a wrong sign or weight, a wrong index range, a
wrong tie-break. If some mutant passed every pin, the pins would not be strong
enough to trust the oracle; this test fails in that case.
"""
import math

import numpy as np
import pytest

import oracle_pins as pins
from oracle import rkv_oracle as orc

_orig_probs = orc.attention_probs
_orig_red = orc.redundancy
_orig_imp = orc.importance
_orig_select = orc.select
_orig_rows = orc.redundancy_rows
_orig_paged = orc.compress_paged


def _paged_shared_variant(K_pages, V_pages, page_table, seq_len, budget, Q, free_list, window,
                          lam, page_size, shared_heads=False, mode="ignored", **variant):
    """Paged compression with one mistake in its head-shared mode."""
    if not shared_heads:
        return _orig_paged(K_pages, V_pages, page_table, seq_len, budget, Q, free_list, window,
                           lam, page_size, **variant)
    if mode == "ignored":                    # every head selects alone
        return _orig_paged(K_pages, V_pages, page_table, seq_len, budget, Q, free_list, window,
                           lam, page_size, **variant)
    # the right selection, but every head's slots receive head 0's rows
    out = _orig_paged(K_pages, V_pages, page_table, seq_len, budget, Q, free_list, window, lam,
                      page_size, shared_heads=True, **variant)
    for s, n in enumerate(seq_len):
        n = int(n)
        if n <= int(budget[s]):
            continue
        kept = out["kept"][s][0]
        K0 = orc.logical_rows(K_pages, page_table[s], n, 0, page_size)
        r = np.arange(len(kept))
        for h in range(1, np.shape(K_pages)[1]):
            out["K_pages"][page_table[s][r // page_size], h, r % page_size] = K0[kept]
    return out


def _pages_variant(page_table, seq_len, budget, free_list, page_size, mode):
    """Page return with one mistake."""
    table = np.array(page_table, copy=True)
    freed = [int(x) for x in free_list]
    todo = []
    for s in range(table.shape[0]):
        n, b = int(seq_len[s]), int(budget[s])
        if n <= b:
            continue
        first = b // page_size + (1 if mode == "first_page_late" else 0)
        end = n // page_size if mode == "floor_of_length" else (n + page_size - 1) // page_size
        ps_ = list(range(first, end))
        if mode == "descending":
            ps_ = ps_[::-1]
        todo += [(s, p) for p in ps_]
    if mode == "page_major":
        todo.sort(key=lambda sp: (sp[1], sp[0]))
    for s, p in todo:
        freed.append(int(table[s, p]))
        if mode == "freed_per_head":        # one append for each of two heads
            freed.append(int(table[s, p]))
        if mode != "entries_kept":
            table[s, p] = -1
    return table, np.asarray(freed, dtype=np.int64)


def _rows_variant(K, rows, symmetric=False, mode="self"):
    R = _orig_red(K, symmetric=symmetric)
    if mode == "shifted":
        return R[np.maximum(np.asarray(rows, dtype=np.int64) - 1, 0)]
    K = np.asarray(K, dtype=np.float64)
    nrm = np.sqrt((K * K).sum(1))
    out = []
    for i in rows:
        i = int(i)
        c = K[:i + 1] @ K[i] / (nrm[:i + 1] * nrm[i])
        out.append(c.max())
    return np.array(out)


def _probs_variant(K, Q, window, mask_shift=0, scale_pow=0.5, causal=True, swap_r=False):
    K = np.asarray(K, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    n, d = K.shape
    g, w, _ = Q.shape
    logits = (Q.reshape(g * w, d) @ K.T / d ** scale_pow).reshape(g, w, n)
    rr = np.arange(w)[::-1] if swap_r else np.arange(w)
    if causal:
        vis = np.arange(n)[None, :] <= (n - w + rr + mask_shift)[:, None]
        logits = np.where(vis[None], logits, -np.inf)
    m = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=2, keepdims=True)


def _red_variant(K, mode):
    K = np.asarray(K, dtype=np.float64)
    n = K.shape[0]
    nrm = np.sqrt((K * K).sum(1))
    C = (K @ K.T) / np.outer(nrm, nrm)
    R = np.zeros(n)
    for i in range(n):
        if mode == "self":
            R[i] = C[i, :i + 1].max()
        elif mode == "later":
            R[i] = C[i, i + 1:].max() if i + 1 < n else 0.0
        elif mode == "mean":
            R[i] = C[i, :i].mean() if i else 0.0
        elif mode == "unnormalised":
            R[i] = (K[:i] @ K[i]).max() if i else 0.0
        elif mode == "symmetric":
            R[i] = np.delete(C[i], i).max()
        elif mode == "all":
            R[i] = C[i].max()
    return R


def _shared_variant(K, V, Q, budget, window, lam, mode, **variant):
    """Head-shared selection with a wrong reduction over heads."""
    K = np.asarray(K)
    V = np.asarray(V)
    n = K.shape[1]
    if n <= budget:
        kept = np.arange(n)
        return dict(kept=kept, K_out=K[:, kept], V_out=V[:, kept], Z=None, Z_sum=None)
    Z = np.stack([orc.scores_head(K[h], Q[h], window, lam, **variant)[2] for h in range(K.shape[0])])
    agg = {"first_head": Z[0], "max_over_heads": Z.max(axis=0), "min_over_heads": Z.min(axis=0)}[mode]
    kept = _orig_select(agg, n, budget, window)
    return dict(kept=kept, K_out=K[:, kept], V_out=V[:, kept], Z=Z, Z_sum=agg)


def _select_variant(Z, n, budget, window, mode):
    if budget <= window:
        raise ValueError
    if n <= budget:
        return np.arange(n)
    Z = np.asarray(Z, dtype=np.float64)
    idx = np.arange(n)
    if mode == "no_window":
        order = np.lexsort((idx, -Z))
        return np.sort(order[:budget])
    cand = n - window
    if mode == "tie_high":
        order = np.lexsort((-idx[:cand], -Z[:cand]))
    elif mode == "lowest":
        order = np.lexsort((idx[:cand], Z[:cand]))
    return np.sort(np.concatenate([order[:budget - window], np.arange(cand, n)]))


MUTANTS = {
    "mean_pool_over_heads": ("importance", lambda K, Q, w, **kw: orc.attention_probs(K, Q, w).mean(1).mean(0)),
    "sum_over_queries": ("importance", lambda K, Q, w, **kw: orc.attention_probs(K, Q, w).sum(1).max(0)),
    "pool_order_swapped": ("importance", lambda K, Q, w, **kw: orc.attention_probs(K, Q, w).max(1).mean(0)),
    "no_causal_mask": ("attention_probs", lambda K, Q, w, **kw: _probs_variant(K, Q, w, causal=False)),
    "mask_off_by_one": ("attention_probs", lambda K, Q, w, **kw: _probs_variant(K, Q, w, mask_shift=1)),
    "mask_reversed": ("attention_probs", lambda K, Q, w, **kw: _probs_variant(K, Q, w, swap_r=True)),
    "scale_1_over_d": ("attention_probs", lambda K, Q, w, **kw: _probs_variant(K, Q, w, scale_pow=1.0)),
    "no_scale": ("attention_probs", lambda K, Q, w, **kw: _probs_variant(K, Q, w, scale_pow=0.0)),
    "red_includes_self": ("redundancy", lambda K, **kw: _red_variant(K, "self")),
    "red_later_tokens": ("redundancy", lambda K, **kw: _red_variant(K, "later")),
    "red_mean": ("redundancy", lambda K, **kw: _red_variant(K, "mean")),
    "red_unnormalised": ("redundancy", lambda K, **kw: _red_variant(K, "unnormalised")),
    "red_symmetric": ("redundancy", lambda K, **kw: _red_variant(K, "symmetric")),
    "z_sign_flipped": ("joint_score", lambda I, R, lam: lam * np.asarray(I) + (1 - lam) * np.asarray(R)),
    "z_weights_swapped": ("joint_score", lambda I, R, lam: (1 - lam) * np.asarray(I) - lam * np.asarray(R)),
    "window_not_protected": ("select", lambda Z, n, b, w: _select_variant(Z, n, b, w, "no_window")),
    "ties_to_larger_index": ("select", lambda Z, n, b, w: _select_variant(Z, n, b, w, "tie_high")),
    "keeps_lowest": ("select", lambda Z, n, b, w: _select_variant(Z, n, b, w, "lowest")),
    # reading variants and head-shared selection
    "symmetric_ignored": ("redundancy", lambda K, symmetric=False: _orig_red(K)),
    "symmetric_includes_self": ("redundancy", lambda K, symmetric=False:
                                _red_variant(K, "all") if symmetric else _orig_red(K)),
    "symmetric_later_only": ("redundancy", lambda K, symmetric=False:
                             _red_variant(K, "later") if symmetric else _orig_red(K)),
    "unmasked_ignored": ("attention_probs", lambda K, Q, w, causal=True: _orig_probs(K, Q, w)),
    "unmasked_off_by_one": ("attention_probs", lambda K, Q, w, causal=True:
                            _orig_probs(K, Q, w) if causal else _probs_variant(K, Q, w, mask_shift=w - 2)),
    "mean_pool_ignored": ("importance", lambda K, Q, w, causal=True, pool="max":
                          _orig_imp(K, Q, w, causal=causal)),
    "mean_pool_sums": ("importance", lambda K, Q, w, causal=True, pool="max":
                       _orig_probs(K, Q, w, causal=causal).mean(1).sum(0) if pool == "mean"
                       else _orig_imp(K, Q, w, causal=causal)),
    "shared_first_head": ("compress_shared", lambda *a, **kw: _shared_variant(*a, mode="first_head", **kw)),
    "shared_max_over_heads": ("compress_shared", lambda *a, **kw: _shared_variant(*a, mode="max_over_heads", **kw)),
    "shared_min_over_heads": ("compress_shared", lambda *a, **kw: _shared_variant(*a, mode="min_over_heads", **kw)),
    # paged page return
    "pages_first_page_late": ("return_pages", lambda *a: _pages_variant(*a, mode="first_page_late")),
    "pages_floor_of_length": ("return_pages", lambda *a: _pages_variant(*a, mode="floor_of_length")),
    "pages_descending": ("return_pages", lambda *a: _pages_variant(*a, mode="descending")),
    "pages_page_major_order": ("return_pages", lambda *a: _pages_variant(*a, mode="page_major")),
    "pages_freed_per_head": ("return_pages", lambda *a: _pages_variant(*a, mode="freed_per_head")),
    "pages_entries_kept": ("return_pages", lambda *a: _pages_variant(*a, mode="entries_kept")),
    # head-shared selection on pages
    "paged_shared_ignored": ("compress_paged", lambda *a, **kw: _paged_shared_variant(*a, mode="ignored", **kw)),
    "paged_shared_head0_rows": ("compress_paged", lambda *a, **kw: _paged_shared_variant(*a, mode="head0_rows", **kw)),
    # redundancy of listed rows
    "rows_include_self": ("redundancy_rows", lambda K, rows, symmetric=False:
                          _rows_variant(K, rows, symmetric, "self")),
    "rows_shifted": ("redundancy_rows", lambda K, rows, symmetric=False:
                     _rows_variant(K, rows, symmetric, "shifted")),
}


def _some_pin_fails():
    for check in pins.ALL_CHECKS:
        for seed in range(3):
            try:
                check(seed)
            except (AssertionError, ValueError, IndexError):
                return check.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = _some_pin_fails()
    assert caught is not None, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_all_pins():
    assert _some_pin_fails() is None
