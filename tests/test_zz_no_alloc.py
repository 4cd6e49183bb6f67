"""rkv_compress_static (no workspace argument, no allocation) against
rkv_compress on the same inputs, on the GPU.

Each case makes two calls in a row through the static entry point, the second
on a smaller input, so the second runs on scratch the first left behind. The
shapes are ones whose kernels use the workspace: long bf16 units (statistics
pass + long-unit kernel + selection + gather), fp32 units (statistics pass +
team kernel), and head-shared selection (summed scores).
"""
import numpy as np
import pytest

import parity as par
from synth import dense_case_host

pytestmark = pytest.mark.gpu

# (seed, N, B, w, G, dtype, units, select_group): first call, then a smaller one
CASES = {
    "long-bf16": ((31, 8000, 6000, 8, 4, "bf16", 2, 1), (32, 7777, 6000, 8, 4, "bf16", 1, 1)),
    "fp32": ((33, 300, 200, 8, 2, "f32", 3, 1), (34, 260, 100, 8, 6, "f32", 1, 1)),
    "shared": ((35, 1152, 1024, 8, 4, "bf16", 4, 2), (36, 600, 500, 8, 4, "bf16", 2, 2)),
}


@pytest.fixture(scope="module")
def rkv():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    import decode_kv_cache_03_amd as mod
    return mod


def _inputs(spec):
    seed, n, b, w, g, dt, units, group = spec
    case = dense_case_host(seed, 1, 1, units, g, n, b, w, 0.1, dt, 0.4, 0.02)
    return case, [par.to_device(x, dt) for x in (case.K, case.V, case.Q)], group


@pytest.mark.parametrize("name", sorted(CASES))
def test_static_matches_workspace_entry_point(rkv, name):
    import torch
    for step, spec in enumerate(CASES[name]):
        case, (K, V, Q), group = _inputs(spec)
        print(f"no-alloc case {name} call {step}: N={case.n} B={case.budget} units={case.num_heads} "
              f"group={group} dtype={case.dtype}", flush=True)
        ref = rkv.compress(K, V, Q, case.budget, case.window, case.lam, debug=True,
                           select_group=group)
        bh, n, b = case.num_heads, case.n, case.budget
        out = dict(K_out=torch.empty((bh, b, 128), dtype=K.dtype, device="cuda"),
                   V_out=torch.empty((bh, b, 128), dtype=K.dtype, device="cuda"),
                   kept_idx=torch.empty((bh, b), dtype=torch.int32, device="cuda"),
                   I=torch.empty((bh, n), dtype=torch.float32, device="cuda"),
                   R=torch.empty((bh, n), dtype=torch.float32, device="cuda"),
                   Z=torch.empty((bh, n), dtype=torch.float32, device="cuda"))
        res = rkv.compress_static(K, V, Q, case.budget, case.window, case.lam,
                                  select_group=group, **out)
        torch.cuda.synchronize()
        assert torch.equal(res.kept_idx, ref.kept_idx), f"{name} call {step}: kept"
        assert par.bits_equal(res.K_out, ref.K_out), f"{name} call {step}: K_out"
        assert par.bits_equal(res.V_out, ref.V_out), f"{name} call {step}: V_out"
        for what, tol in (("I", par.TOL_I), ("R", par.TOL_RZ), ("Z", par.TOL_RZ)):
            a = getattr(res, what).cpu().numpy().ravel()
            r = getattr(ref, what).cpu().numpy().ravel()
            par.assert_close(a, r, tol, f"{name} call {step}: {what}")
