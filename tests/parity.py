"""Helpers for comparing the HIP path with the oracle (used by the gpu tests).

Tolerances (scores are computed in fp32 on the GPU, fp64 in the oracle):
  I: |gpu - ref| <= 1e-3 * |ref| + 1e-7
  R, Z: |gpu - ref| <= 1e-3 * |ref| + 1e-5
The relative bound is the target stated for the scores. The absolute floors
cover values near zero, where a relative bound is meaningless: a cosine is
an fp32-accumulated dot product of 128 exact products, whose error is at most
128 * 2^-24 * sum|k_i,d k_j,d| / (|k_i| |k_j|) <= 7.7e-6 (Cauchy-Schwarz),
plus a few ulp from the fp32 norms; I is a probability (<= 1) whose fp32
softmax error is a few ulp of its magnitude.

Kept sets (tau = 1e-4): |kept| = min(N, B); the window is kept; indices
ascend; and for every kept non-window i and evicted j, Z_ref(i) >= Z_ref(j)
- tau. This equals the oracle's set exactly whenever the oracle's k-th and
(k+1)-th best scores differ by more than tau, and otherwise admits only
swaps among scores within tau of the boundary.
Compacted rows are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

from oracle import rkv_oracle as orc

TAU = 1e-4
TOL_I = (1e-3, 1e-7)
TOL_RZ = (1e-3, 1e-5)


def assert_close(gpu, ref, tol, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = tol[0] * np.abs(ref) + tol[1]
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{what}: {bad.size} entries out of tolerance, first at {bad[:5]}: "
                           f"gpu={gpu[bad[:5]]} ref={ref[bad[:5]]}")


def assert_tau_valid(kept_gpu, z_ref, n, budget, window, what=""):
    kept = np.asarray(kept_gpu, dtype=np.int64)
    nkeep = min(n, budget)
    assert kept.shape == (nkeep,), (what, kept.shape, nkeep)
    assert np.all(np.diff(kept) > 0), f"{what}: kept not strictly ascending"
    assert kept[0] >= 0 and kept[-1] < n, what
    if n <= budget:
        assert np.array_equal(kept, np.arange(n)), what
        return
    assert set(range(n - window, n)) <= set(kept.tolist()), f"{what}: window not kept"
    cand = n - window
    kmask = np.zeros(n, dtype=bool)
    kmask[kept] = True
    kept_nw = np.nonzero(kmask[:cand])[0]
    evicted = np.nonzero(~kmask[:cand])[0]
    assert kept_nw.size == budget - window, what
    zmin_kept = z_ref[kept_nw].min()
    zmax_ev = z_ref[evicted].max()
    assert zmin_kept >= zmax_ev - TAU, (f"{what}: kept score {zmin_kept} below evicted "
                                        f"{zmax_ev} by more than tau")
    srt = np.sort(z_ref[:cand])[::-1]
    k = budget - window
    if srt[k - 1] - srt[k] > TAU:
        ref_kept = orc.select(z_ref, n, budget, window)
        assert np.array_equal(kept, ref_kept), f"{what}: strict case differs from oracle"


def check_head(K, V, Q, budget, window, lam, kept, K_out, V_out, I=None, R=None, Z=None,
               what="", ref=None):
    """Check one unit's GPU outputs (numpy) against the oracle."""
    n = K.shape[0]
    ref = ref if ref is not None else orc.compress_head(K, V, Q, budget, window, lam)
    if n > budget:
        if I is not None:
            assert_close(I, ref["I"], TOL_I, f"{what} I")
        if R is not None:
            assert_close(R, ref["R"], TOL_RZ, f"{what} R")
        if Z is not None:
            assert_close(Z, ref["Z"], TOL_RZ, f"{what} Z")
        assert_tau_valid(kept, ref["Z"], n, budget, window, what)
    else:
        assert np.array_equal(np.asarray(kept), np.arange(n)), what
    kept = np.asarray(kept, dtype=np.int64)
    # float32 images of the rows: exact and injective for bf16 and fp32 data
    assert np.array_equal(np.ascontiguousarray(K_out, np.float32).view(np.uint32),
                          np.ascontiguousarray(K[kept], np.float32).view(np.uint32)), \
        f"{what}: K_out is not K[kept]"
    assert np.array_equal(np.ascontiguousarray(V_out, np.float32).view(np.uint32),
                          np.ascontiguousarray(V[kept], np.float32).view(np.uint32)), \
        f"{what}: V_out is not V[kept]"
    if np.array_equal(kept, ref["kept"]):
        assert np.array_equal(K_out, ref["K_out"]) and np.array_equal(V_out, ref["V_out"])
    return ref


def to_device(x, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def to_host_f32(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def bits_equal(a, b) -> bool:
    """Bitwise equality of two torch tensors of the same dtype."""
    import torch
    if a.dtype == torch.bfloat16:
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
    return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
