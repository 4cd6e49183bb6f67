"""The oracle against the pure-Python brute force on tiny heads drawn by
hypothesis (N <= 12, d <= 16, G <= 3, w <= 4), under every reading variant,
and head-shared selection on pairs of such heads. CPU only."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import bruteforce as bf
from oracle import rkv_oracle as orc


@st.composite
def tiny_heads(draw, heads=1):
    n = draw(st.integers(4, 12))
    d = draw(st.integers(2, 16))
    g = draw(st.integers(1, 3))
    w = draw(st.integers(1, min(4, n - 2)))
    b = draw(st.integers(w + 1, n - 1))
    lam = draw(st.sampled_from([0.0, 0.1, 0.5, 0.9, 1.0]))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((heads, n, d))
    if draw(st.booleans()):            # plant an exact copy (scaled) of an earlier key
        j = int(rng.integers(1, n))
        K[:, j] = 2.0 * K[:, int(rng.integers(0, j))]
    V = rng.standard_normal((heads, n, d))
    Q = draw(st.sampled_from([0.0, 1.0, 3.0])) * rng.standard_normal((heads, g, w, d))
    variant = dict(symmetric=draw(st.booleans()), causal=draw(st.booleans()),
                   pool=draw(st.sampled_from(["max", "mean"])))
    return K, V, Q, b, w, lam, variant


def _same_selection(kept_o, kept_r, Z, n, b, w):
    """Equal kept sets; where the b-w-th and next best scores lie within
    rounding of each other, both sets only need to be valid for Z."""
    Z = np.asarray(Z, dtype=np.float64)
    srt = np.sort(Z[:n - w])[::-1]
    if srt[b - w - 1] - srt[b - w] > 1e-9:
        assert list(kept_o) == list(kept_r)
        return
    for kept in (kept_o, kept_r):
        kept = set(int(i) for i in kept)
        assert set(range(n - w, n)) <= kept and len(kept) == b
        ins = [Z[i] for i in kept if i < n - w]
        outs = [Z[i] for i in range(n - w) if i not in kept]
        assert min(ins) >= max(outs) - 1e-9


def _close(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.abs(a - b) <= 1e-12 * np.maximum(1.0, np.abs(b)))


@settings(max_examples=80, deadline=None, derandomize=True)
@given(tiny_heads())
def test_oracle_matches_bruteforce(case):
    K, V, Q, b, w, lam, variant = case
    o = orc.compress_head(K[0], V[0], Q[0], b, w, lam, **variant)
    r = bf.compress_head_bf(K[0].tolist(), V[0].tolist(), Q[0].tolist(), b, w, lam, **variant)
    _close(o["I"], r["I"])
    _close(o["R"], r["R"])
    _close(o["Z"], r["Z"])
    _same_selection(o["kept"], r["kept"], r["Z"], K.shape[1], b, w)


@settings(max_examples=40, deadline=None, derandomize=True)
@given(tiny_heads(heads=2))
def test_shared_selection_matches_bruteforce(case):
    K, V, Q, b, w, lam, variant = case
    o = orc.compress_shared(K, V, Q, b, w, lam, **variant)
    r = bf.compress_shared_bf(K.tolist(), V.tolist(), Q.tolist(), b, w, lam, **variant)
    _same_selection(o["kept"], r["kept"], np.sum(r["Z"], axis=0), K.shape[1], b, w)
