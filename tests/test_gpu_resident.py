"""GPU parity of the register-resident dense kernel (rkv_k2_resident, through the C ABI).

Dense bf16 units of at most 1024 + 128 candidates whose GQA group and window
fill at most one 32-row query block take this kernel: the first N-128 keys
are held in registers and every key is read once. Cases cover a ragged last
tile, a last tile of one row, a single tile, exact tile multiples, every
window/group split that fits one query block, and the importance variants
(no causal window, mean pooling). Each case also checks that the call ran
this kernel (its launch label in the library's timing records).
"""
import numpy as np
import pytest

import parity as par
from oracle import rkv_oracle as orc
from synth import dense_case_host

pytestmark = pytest.mark.gpu

SHAPES = [
    # (N, B, w, G, heads)
    (1152, 1024, 8, 4, 3),    # the Llama3-8B event shape: 9 tiles, 8 held
    (1100, 1000, 8, 4, 2),    # ragged last tile
    (1025, 1000, 8, 4, 2),    # last tile of one row
    (1024, 900, 8, 4, 2),     # 8 whole tiles
    (129, 100, 8, 4, 2),      # one held tile and a one-row last tile
    (128, 100, 8, 4, 2),      # a single whole tile, nothing held
    (70, 40, 8, 4, 2),        # a single partial tile
    (600, 300, 4, 3, 2),      # 4 window rows padded to 8 per head, 3 heads
    (500, 300, 16, 2, 2),     # 16 rows per head
    (400, 200, 32, 1, 2),     # one head of 32 window rows
    (300, 200, 1, 4, 2),      # a window of one query
    (700, 520, 6, 4, 2),      # window padded to 8 rows per head
]

VARIANTS = {
    "default": {},
    "no-causal": dict(causal=False),
    "pool-mean": dict(pool="mean"),
    "both": dict(causal=False, pool="mean"),
}


@pytest.fixture(scope="module")
def rkv():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    import decode_kv_cache_03_amd as mod
    return mod


def _run(rkv, case, **kw):
    import torch
    K = par.to_device(case.K, case.dtype)
    V = par.to_device(case.V, case.dtype)
    Q = par.to_device(case.Q, case.dtype)
    torch.cuda.synchronize()
    rkv.timing_enable(True)
    res = rkv.compress(K, V, Q, case.budget, case.window, case.lam, debug=True, **kw)
    torch.cuda.synchronize()
    labels = rkv.timing_read()
    rkv.timing_enable(False)
    return res, labels


def _check(rkv, case, var, what):
    res, labels = _run(rkv, case, **var)
    assert list(labels) == ["rkv_k2_resident"], f"{what}: launched {sorted(labels)}"
    n, b, w, lam = case.n, case.budget, case.window, case.lam
    kept = res.kept_idx.cpu().numpy()
    Ko, Vo = par.to_host_f32(res.K_out), par.to_host_f32(res.V_out)
    I, R, Z = (t.cpu().numpy() for t in (res.I, res.R, res.Z))
    for h in range(case.num_heads):
        ref = orc.compress_head(case.K[h], case.V[h], case.Q[h], b, w, lam, **var)
        par.check_head(case.K[h], case.V[h], case.Q[h], b, w, lam, kept[h], Ko[h], Vo[h],
                       I[h], R[h], Z[h], what=f"{what} head {h}", ref=ref)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"N{s[0]}-B{s[1]}-w{s[2]}-G{s[3]}" for s in SHAPES])
def test_resident_default(rkv, shape):
    n, b, w, g, heads = shape
    case = dense_case_host(101 + n, 1, 1, heads, g, n, b, w, 0.1, "bf16", 0.4, 0.02)
    _check(rkv, case, {}, f"{shape}")


@pytest.mark.parametrize("variant", ["no-causal", "pool-mean", "both"])
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[1], SHAPES[7], SHAPES[10]],
                         ids=lambda s: f"N{s[0]}-w{s[2]}-G{s[3]}")
def test_resident_variants(rkv, shape, variant):
    n, b, w, g, heads = shape
    case = dense_case_host(201 + n, 1, 1, heads, g, n, b, w, 0.1, "bf16", 0.4, 0.02)
    _check(rkv, case, VARIANTS[variant], f"{shape} {variant}")


@pytest.mark.parametrize("lam", [0.0, 1.0])
def test_resident_lambda_ends(rkv, lam):
    """lambda = 0: Z = -R exactly (selection by redundancy alone); lambda = 1:
    Z = I exactly."""
    case = dense_case_host(303, 1, 1, 2, 4, 1152, 1024, 8, lam, "bf16", 0.4, 0.02)
    _check(rkv, case, {}, f"lambda {lam}")
    res, _ = _run(rkv, case)
    Z, R, I = (t.cpu().numpy() for t in (res.Z, res.R, res.I))
    if lam == 0.0:
        assert np.array_equal(Z, -R + 0.0)
    else:
        assert np.array_equal(Z, I + 0.0)


def test_resident_units_beyond_grid(rkv):
    """More units than CUs: every workgroup runs several units back to back
    (the tile stream and query slots carry over between them)."""
    import torch
    units = 700
    case = dense_case_host(404, 1, 1, units, 4, 1100, 1000, 8, 0.1, "bf16", 0.4, 0.02)
    res, labels = _run(rkv, case)
    assert list(labels) == ["rkv_k2_resident"]
    kept = res.kept_idx.cpu().numpy()
    Z = res.Z.cpu().numpy()
    Ko = par.to_host_f32(res.K_out)
    for u in (0, 255, 256, 511, 512, 699):
        ref = orc.compress_head(case.K[u], case.V[u], case.Q[u], case.budget, case.window, case.lam)
        par.assert_close(Z[u], ref["Z"], par.TOL_RZ, f"unit {u} Z")
        par.assert_tau_valid(kept[u], ref["Z"], case.n, case.budget, case.window, f"unit {u}")
        assert np.array_equal(Ko[u], case.K[u][kept[u].astype(np.int64)]), f"unit {u} rows"
    torch.cuda.synchronize()


TIE_CASES = [
    # (name, N, B, w, lambda): keys drawn from few distinct rows, so many
    # candidates share the same Z exactly and the index order decides
    ("one-row", 1152, 1024, 8, 0.0),
    ("one-row-lam", 1152, 1024, 8, 0.1),
    ("three-rows", 1100, 700, 8, 0.0),
    ("two-rows-small", 300, 150, 8, 0.0),
    # the two-pass kernel (1152 < N <= 2176): its selection over 2168 and
    # 1992 candidates, rows below 1024 moved a unit later
    ("one-row-2pass", 2176, 2048, 8, 0.0),
    ("three-rows-2pass", 2000, 1504, 8, 0.1),
]


@pytest.mark.parametrize("case_", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_resident_selection_ties(rkv, case_):
    """Exact ties: the kept set must be the selection of the device's own Z
    with ties to the smaller index (the oracle's select on those values)."""
    name, n, b, w, lam = case_
    rows = 1 if name.startswith("one") else (3 if name.startswith("three") else 2)
    case = dense_case_host(505 + n + rows, 1, 1, 4, 4, n, b, w, lam, "bf16", 0.0, 0.02)
    rng = np.random.default_rng(505 + rows)
    for h in range(case.num_heads):
        pick = rng.integers(0, rows, size=n)
        base = case.K[h, :rows].copy()
        case.K[h] = base[pick]
    res, labels = _run(rkv, case)
    assert list(labels) == ["rkv_k2_resident" if n <= 1152 else "rkv_k2_resident2"]
    kept = res.kept_idx.cpu().numpy()
    Z = res.Z.cpu().numpy()
    Ko = par.to_host_f32(res.K_out)
    for h in range(case.num_heads):
        z = Z[h].astype(np.float64)
        assert len(np.unique(z[: n - w])) < n // 4, f"{name}: expected many tied scores"
        assert np.array_equal(kept[h], orc.select(z, n, b, w)), f"{name} head {h}: kept set"
        assert np.array_equal(Ko[h], case.K[h][kept[h].astype(np.int64)]), f"{name} head {h}: rows"
