"""GPU parity of the reading variants and of head-shared selection (through the C ABI).

Variants: symmetric redundancy (max over every other candidate), importance
without the in-window causal mask, and mean instead of max pooling over the
GQA heads, alone and together, on the fused dense bf16 kernel, the
workgroup-team path (fp32, and bf16 units too long for the fused kernel) and
the paged path. Head-shared selection: runs of consecutive units select once
on the sum of their scores; checked against the oracle's compress_shared.
"""
import numpy as np
import pytest

import parity as par
from oracle import rkv_oracle as orc
from synth import CONFIGS, dense_case_device, dense_case_host, paged_case_host

pytestmark = pytest.mark.gpu

VARIANTS = {
    "symmetric": dict(symmetric=True),
    "no-causal": dict(causal=False),
    "pool-mean": dict(pool="mean"),
    "all": dict(symmetric=True, causal=False, pool="mean"),
}

SHAPES = [
    # (N, B, w, G, lam, dtype, heads)
    (700, 512, 8, 5, 0.1, "bf16", 2),      # fused kernel, ragged last tile
    (1152, 1024, 8, 4, 0.1, "bf16", 2),    # fused kernel, the Llama3-8B event shape
    (70, 40, 8, 4, 0.1, "bf16", 2),        # one partial tile
    (300, 200, 8, 2, 0.1, "f32", 2),       # team path (fp32)
    (8000, 6000, 8, 4, 0.1, "bf16", 1),    # team path (unit too long for the fused kernel)
    (2176, 2048, 8, 5, 0.1, "bf16", 2),    # two-pass resident kernel (symmetric: fused kernel)
]


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
    res = rkv.compress(K, V, Q, case.budget, case.window, case.lam, debug=True, **kw)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("shape", SHAPES, ids=[f"N{s[0]}-B{s[1]}-G{s[3]}-{s[5]}" for s in SHAPES])
def test_dense_variants(rkv, shape, variant):
    n, b, w, g, lam, dt, heads = shape
    var = VARIANTS[variant]
    case = dense_case_host(31 + n, 1, 1, heads, g, n, b, w, lam, dt, 0.4, 0.02)
    res = _run(rkv, case, **var)
    kept = res.kept_idx.cpu().numpy()
    Ko, Vo = par.to_host_f32(res.K_out), par.to_host_f32(res.V_out)
    I, R, Z = (t.cpu().numpy() for t in (res.I, res.R, res.Z))
    for h in range(heads):
        ref = orc.compress_head(case.K[h], case.V[h], case.Q[h], b, w, lam, **var)
        par.check_head(case.K[h], case.V[h], case.Q[h], b, w, lam, kept[h], Ko[h], Vo[h],
                       I[h], R[h], Z[h], what=f"{shape} {variant} head {h}", ref=ref)


def test_symmetric_scores_both_copies(rkv):
    """Exact copies (up to a power-of-two scale): under the symmetric reading
    the source and the copy both reach cosine 1; under the default only the
    copy does."""
    case = dense_case_host(41, 1, 1, 2, 4, 600, 480, 8, 0.0, "bf16", coverage=0.0)
    rng = np.random.default_rng(41)
    pairs = [(int(a), int(c)) for a, c in zip(rng.choice(np.arange(0, 280), 40, replace=False),
                                              rng.choice(np.arange(300, 590), 40, replace=False))]
    for h in range(case.num_heads):
        for a, c in pairs:
            case.K[h, c] = case.K[h, a] * np.float32(2.0)
    R_sym = _run(rkv, case, symmetric=True).R.cpu().numpy()
    R_def = _run(rkv, case).R.cpu().numpy()
    src = [a for a, _ in pairs]
    cpy = [c for _, c in pairs]
    assert np.all(np.abs(R_sym[:, src] - 1.0) <= 1e-5)
    assert np.all(np.abs(R_sym[:, cpy] - 1.0) <= 1e-5)
    assert np.all(np.abs(R_def[:, cpy] - 1.0) <= 1e-5)
    assert np.all(R_def[:, src] < 0.9)
    assert np.all(R_sym >= R_def - 1e-6)


# symmetric (and all) run the 512-row long-unit form on the pages; no-causal
# and mean pooling the 1024-row form
@pytest.mark.parametrize("variant", ["symmetric", "no-causal", "pool-mean", "all"])
def test_paged_variants(rkv, variant):
    import torch
    var = VARIANTS[variant]
    lens, fracs = [40, 100, 16, 130, 300, 520], [0.5, 0.3, 0.9, 0.4, 0.25, 0.1]
    case = paged_case_host(51, lens, fracs, kv_heads=2, gqa=2, window=8, lam=0.1)
    Kp = par.to_device(case.K_pages, case.dtype)
    Vp = par.to_device(case.V_pages, case.dtype)
    table = torch.from_numpy(case.page_table).cuda()
    ref = orc.compress_paged(case.K_pages, case.V_pages, case.page_table, case.seq_len,
                             case.budget, case.Q, case.free_list, case.window, case.lam,
                             case.page_size, **var)
    cap = len(ref["free_list"])
    fl = torch.full((cap,), -5, dtype=torch.int32, device="cuda")
    fl[:len(case.free_list)] = torch.from_numpy(case.free_list.astype(np.int32)).cuda()
    res = rkv.compress_paged(Kp, Vp, table, case.seq_len, case.budget, par.to_device(case.Q, case.dtype),
                             fl, len(case.free_list), case.window, case.lam, debug=True, **var)
    torch.cuda.synchronize()
    assert np.array_equal(table.cpu().numpy(), ref["page_table"])
    assert np.array_equal(fl.cpu().numpy(), ref["free_list"].astype(np.int32))
    H, ps = case.kv_heads, case.page_size
    kept_all = res.kept_idx.cpu().numpy()
    Z_all = res.Z.cpu().numpy()
    Kn = par.to_host_f32(Kp)
    k = z = 0
    for s, (n, b) in enumerate(zip(case.seq_len, case.budget)):
        n, b = int(n), int(b)
        nk = min(n, b)
        for h in range(H):
            kept = kept_all[k + h * nk: k + (h + 1) * nk].astype(np.int64)
            what = f"{variant} seq {s} head {h}"
            if n > b:
                Kl = orc.logical_rows(case.K_pages, case.page_table[s], n, h, ps)
                rr = orc.compress_head(Kl, Kl, case.Q[s, h], b, case.window, case.lam, **var)
                par.assert_close(Z_all[z + h * n: z + (h + 1) * n], rr["Z"], par.TOL_RZ, what + " Z")
                par.assert_tau_valid(kept, rr["Z"], n, b, case.window, what)
                r = np.arange(nk)
                assert np.array_equal(Kn[case.page_table[s][r // ps], h, r % ps], Kl[kept]), what
            else:
                assert np.array_equal(kept, np.arange(n)), what
        k += H * nk
        z += H * n


def _check_shared(case, res, group, var, groups=None, what=""):
    """Every unit of a group keeps the same indices; they are tau-valid for the
    oracle's summed scores; each unit's Z matches its own oracle Z; rows are a
    bit-exact gather."""
    n, b, w = case.n, case.budget, case.window
    kept = res.kept_idx.cpu().numpy()
    Z = res.Z.cpu().numpy()
    Ko, Vo = par.to_host_f32(res.K_out), par.to_host_f32(res.V_out)
    ngroups = case.num_heads // group
    for gi in (range(ngroups) if groups is None else groups):
        u0 = gi * group
        sl = slice(u0, u0 + group)
        ref = orc.compress_shared(case.K[sl], case.V[sl], case.Q[sl], b, w, case.lam, **var)
        for h in range(group):
            u = u0 + h
            assert np.array_equal(kept[u], kept[u0]), f"{what} group {gi}: unit {u} differs"
            par.assert_close(Z[u], ref["Z"][h], par.TOL_RZ, f"{what} unit {u} Z")
            ku = kept[u].astype(np.int64)
            assert np.array_equal(Ko[u], case.K[u][ku]) and np.array_equal(Vo[u], case.V[u][ku]), \
                f"{what} unit {u}: rows are not K[kept]"
        par.assert_tau_valid(kept[u0], ref["Z_sum"], n, b, w, f"{what} group {gi}")


SHARED = [
    # (N, B, w, G, dtype, units, group)
    (1152, 1024, 8, 4, "bf16", 8, 8),      # one layer of Llama3-8B: its 8 KV heads share
    (700, 512, 8, 5, "bf16", 16, 4),       # several groups, ragged tile
    (300, 200, 8, 2, "f32", 4, 2),         # team path
    (8000, 6000, 8, 4, "bf16", 2, 2),      # team path, long units
    (2176, 2048, 8, 5, "bf16", 4, 2),      # two-pass resident kernel, scores only
]


@pytest.mark.parametrize("variant", ["default", "all"])
@pytest.mark.parametrize("shape", SHARED, ids=[f"N{s[0]}-{s[4]}-u{s[5]}-g{s[6]}" for s in SHARED])
def test_shared_selection(rkv, shape, variant):
    n, b, w, g, dt, units, group = shape
    var = {} if variant == "default" else VARIANTS[variant]
    case = dense_case_host(61 + n, 1, 1, units, g, n, b, w, 0.1, dt, 0.4, 0.02)
    res = _run(rkv, case, select_group=group, **var)
    _check_shared(case, res, group, var, what=f"{shape} {variant}")


def test_shared_selection_full_size(rkv):
    """One Llama3-8B decode event (16384 units) with the 8 KV heads of every
    layer of every sequence sharing one kept set."""
    import torch
    c = CONFIGS[2]
    case = dense_case_device(2, c["batch"], c["layers"], c["kv_heads"], c["gqa"], c["n"],
                             c["budget"], c["window"], c["lam"], c["dtype"], c["coverage"],
                             c["sigma"])
    group = c["kv_heads"]
    res = rkv.compress(case.K, case.V, case.Q, case.budget, case.window, case.lam, debug=True,
                       select_group=group)
    torch.cuda.synchronize()
    n, b, w = case.n, case.budget, case.window
    kept = res.kept_idx
    kg = kept.view(-1, group, b)
    assert torch.equal(kg, kg[:, :1].expand_as(kg))
    assert torch.all(kept[:, 1:] > kept[:, :-1])
    assert torch.all(kept[:, b - w:] == torch.arange(n - w, n, device="cuda", dtype=torch.int32))
    idx = kept.long()[..., None].expand(-1, -1, 128)
    assert par.bits_equal(res.K_out, torch.gather(case.K, 1, idx))
    assert par.bits_equal(res.V_out, torch.gather(case.V, 1, idx))
    # the oracle on two sampled groups
    host = type("HostCase", (), {})()
    for gi in (0, 2047):
        sl = slice(gi * group, (gi + 1) * group)
        host.K, host.V, host.Q = (par.to_host_f32(t[sl]) for t in (case.K, case.V, case.Q))
        host.num_heads, host.n, host.budget, host.window, host.lam = group, n, b, w, case.lam
        sub = type("Res", (), {})()
        sub.kept_idx, sub.Z, sub.K_out, sub.V_out = kept[sl], res.Z[sl], res.K_out[sl], res.V_out[sl]
        _check_shared(host, sub, group, {}, what=f"event group {gi}")
