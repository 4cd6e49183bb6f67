"""CPU model of the paged in-place compaction's order of memory operations
(k5_paged_kernel in decode_kv_cache_03_amd/csrc/k5_compact.hip).

One workgroup moves one (sequence, head): slot r receives row kept[r], for
chunks of 128 slots in ascending order. Within a chunk the threads run in
any order, so the model loads every moved row of the chunk first (the wait
and the barrier), then stores them in a random order. Slots hold row
identities; the final slots must equal the out-of-place gather, and no
store may hit a row that a later chunk still reads. Two planted mistakes
must be caught: a chunk whose rows are stored as soon as each is loaded (no
barrier), and chunks taken in descending order.
"""
import numpy as np
import pytest

CH = 128


def kept_list(rng, N, B, W, kind="random"):
    if kind == "random":
        body = np.sort(rng.choice(N - W, size=B - W, replace=False))
    elif kind == "front":          # every candidate kept up to B-w: nothing moves but the window
        body = np.arange(B - W)
    else:                          # dense runs: sources just past their slots
        body = np.sort(rng.choice(min(N - W, B - W + 40), size=B - W, replace=False))
    return np.concatenate([body, np.arange(N - W, N)]).astype(np.int64)


def compact(kept, N, B, rng, mode="kernel"):
    mem = np.arange(N)
    written = np.zeros(N, dtype=bool)
    starts = list(range(0, B, CH))
    if mode == "descending":
        starts = starts[::-1]
    for c0 in starts:
        rows = [r for r in range(c0, min(c0 + CH, B)) if kept[r] != r]
        for r in rows:                               # reads of this chunk: none already overwritten
            assert 0 <= kept[r] < N and r <= kept[r]
            if mode == "kernel":
                assert not written[kept[r]], "a source read after it was overwritten"
        if mode == "no_barrier":
            for r in rng.permutation(rows):
                mem[r] = mem[kept[r]]
                written[r] = True
            continue
        vals = {r: mem[kept[r]] for r in rows}
        for r in rng.permutation(rows):
            mem[r] = vals[r]
            written[r] = True
    return mem[:B]


CASES = [(2048, 208, 8, "random"), (32768, 11136, 8, "random"), (4000, 3984, 8, "random"),
         (1153, 1024, 8, "random"), (600, 400, 1, "random"), (300, 32, 8, "random"),
         (5000, 1024, 8, "front"), (3000, 1024, 8, "dense"), (257, 256, 8, "dense")]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}-B{c[1]}-{c[3]}" for c in CASES])
def test_in_place_compaction_equals_gather(case):
    N, B, W, kind = case
    rng = np.random.default_rng(N + B)
    for _ in range(3):
        kept = kept_list(rng, N, B, W, kind)
        assert np.array_equal(compact(kept, N, B, rng), kept)


@pytest.mark.parametrize("mode", ["no_barrier", "descending"])
def test_planted_order_mistakes_are_caught(mode):
    rng = np.random.default_rng(11)
    bad = 0
    for N, B, W, kind in CASES:
        kept = kept_list(rng, N, B, W, "dense" if kind == "front" else kind)
        bad += not np.array_equal(compact(kept, N, B, rng, mode), kept)
    assert bad >= 3
