"""CPU model of the resident kernels' online softmax statistics update
(stats_accumulate in decode_kv_cache_03_amd/csrc/rkv_resident.hpp), in
float32 as the device computes it.

The device starts a query column's running max at -FLT_MAX instead of -inf
and drops the tests that skipped an update while nothing was seen. The model
checks that this gives bit-identical (max, sum) pairs to the guarded form on
sequences of logit blocks with masked entries (-inf), fully masked blocks
(also at the start) and extreme values; exp2 is numpy's float32 exp2 on both
sides, so only the control flow differs.
"""
import numpy as np

F32 = np.float32
NO_LOGIT = F32(-3.40282347e38)


def exp2(x):
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        return np.exp2(F32(x), dtype=np.float32)


def sentinel_update(m, s, lg):
    mt = F32(np.max(lg))
    mn = F32(max(m, mt))
    acc = F32(s * exp2(F32(m - mn)))
    for x in lg:
        acc = F32(acc + exp2(F32(x - mn)))
    return mn, acc


def guarded_update(m, s, lg):
    mt = F32(np.max(lg))
    mn = F32(max(m, mt))
    if mn == -np.inf:
        return m, s
    acc = F32(s * exp2(F32(m - mn))) if m != -np.inf else F32(0.0)
    for x in lg:
        acc = F32(acc + exp2(F32(x - mn)))
    return mn, acc


def run(blocks):
    ms, ss = NO_LOGIT, F32(0.0)
    mg, sg = F32(-np.inf), F32(0.0)
    for lg in blocks:
        ms, ss = sentinel_update(ms, ss, lg)
        mg, sg = guarded_update(mg, sg, lg)
    return (ms, ss), (mg, sg)


def test_same_sums_as_the_guarded_update():
    rng = np.random.default_rng(0)
    for trial in range(400):
        nblocks = int(rng.integers(1, 12))
        blocks = []
        for b in range(nblocks):
            lg = (rng.standard_normal(4) * rng.choice([0.1, 3.0, 40.0])).astype(np.float32)
            lg[rng.random(4) < 0.3] = -np.inf
            if rng.random() < 0.2:
                lg[:] = -np.inf                       # a fully masked block
            blocks.append(lg)
        (ms, ss), (mg, sg) = run(blocks)
        assert ss.tobytes() == sg.tobytes(), (trial, ss, sg)
        if sg > 0:                                    # something was seen: the same max
            assert ms.tobytes() == mg.tobytes()
        else:                                         # nothing seen: merged as unseen either way
            assert ss == 0 and mg == -np.inf and ms == NO_LOGIT


def test_first_blocks_masked():
    blocks = [np.full(4, -np.inf, np.float32)] * 3 + [np.array([1.5, -2.0, -np.inf, 0.25], np.float32)]
    (ms, ss), (mg, sg) = run(blocks)
    assert ms == mg == F32(1.5) and ss.tobytes() == sg.tobytes()
