"""CPU model of the workgroup selection with one barrier per digit pass
(select_block_lean in decode_kv_cache_03_amd/csrc/rkv_select.hpp), with a
race check between its waves.

The model runs the device code's steps for every wave of a 512-thread
workgroup (8 waves of 64 lanes), epoch by epoch (an epoch is the code between
two workgroup barriers), and records every LDS access with its epoch, wave,
address and kind (read, write, atomic add). Two accesses to one address in
the same epoch by different waves conflict unless both are reads or both are
atomic adds; any
conflict fails the test, whatever order the waves would run in. The result
(kept list and output row of every candidate) is compared with the oracle's
selection step, and the waves run in a random order per epoch, so a result
that depended on the order would show too. The index logic is modelled lane
by lane: the strided keys read once before the digit passes, the histogram
with the first-lane aggregation, each wave's own scan of the counts, the
packed block scan of the ordered pass.
"""
import numpy as np
import pytest

from oracle import rkv_oracle as orc

NT, LANES = 512, 64
WAVES = NT // LANES


def order_key(z32):
    b = (np.asarray(z32, dtype=np.float32) + np.float32(0.0)).view(np.uint32).astype(np.uint64)
    return np.where(b & 0x80000000, (~b) & 0xFFFFFFFF, b | 0x80000000).astype(np.uint64)


class Lds:
    """Named LDS arrays with access recording."""

    def __init__(self, arrays):
        self.mem = {k: np.array(v, dtype=np.int64) for k, v in arrays.items()}
        self.log = []          # (epoch, wave, array, index, kind)
        self.epoch = 0

    def read(self, wave, name, idx):
        self.log.append((self.epoch, wave, name, int(idx), "r"))
        return int(self.mem[name][idx])

    def write(self, wave, name, idx, val):
        self.log.append((self.epoch, wave, name, int(idx), "w"))
        self.mem[name][idx] = val

    def atomic_add(self, wave, name, idx, val):
        self.log.append((self.epoch, wave, name, int(idx), "a"))
        self.mem[name][idx] += val

    def conflicts(self):
        seen = {}
        bad = []
        for e, w, n, i, kind in self.log:
            for w2, k2 in seen.get((e, n, i), ()):
                if w2 != w and kind + k2 not in ("rr", "aa"):
                    bad.append((e, n, i, w2, k2, w, kind))
            seen.setdefault((e, n, i), set()).add((w, kind))
        return bad


def wave_program(wave, N, B, W, lds, shared, clear_late=False):
    """One wave's steps of select_block_lean; yields at each barrier.
    clear_late: a planted mistake, the next pass's histogram cleared after
    the barrier instead of before it."""
    lane = np.arange(LANES)
    tid = wave * LANES + lane
    cand, k = N - W, B - W
    # each thread's strided candidates wave*64 + lane + j*NT, read once: their
    # keys stay in registers for the digit passes
    kmax = (cand + NT - 1) // NT
    regkey = np.zeros((kmax, LANES), np.uint64)
    for j in range(kmax):
        for l in range(LANES):
            i = wave * LANES + j * NT + l
            if i < cand:
                lds.read(wave, "z", i)
                regkey[j, l] = shared["keys"][i]
    for t in tid[tid < 256]:
        lds.write(wave, "hist0", t, 0)
        lds.write(wave, "hist1", t, 0)
    yield
    prefix, mask, remaining = 0, 0, k
    for pas in range(4):
        shift = 24 - 8 * pas
        hc = f"hist{pas % 3}"
        for j, i0 in enumerate(range(wave * LANES, cand, NT)):
            i = i0 + lane
            valid = i < cand
            key = np.where(valid, regkey[j], 0).astype(np.uint64)
            inn = valid & ((key & mask) == prefix)
            dig = (key >> shift) & 255
            if inn.any():
                lead = int(np.nonzero(inn)[0][0])
                d0 = int(dig[lead])
                same = inn & (dig == d0)
                lds.atomic_add(wave, hc, d0, int(same.sum()))
                for l in np.nonzero(inn & (dig != d0))[0]:
                    lds.atomic_add(wave, hc, int(dig[l]), 1)
        if 1 <= pas < 3 and not clear_late:
            for t in tid[tid < 256]:
                lds.write(wave, f"hist{(pas + 1) % 3}", t, 0)
        yield
        if 1 <= pas < 3 and clear_late:
            for t in tid[tid < 256]:
                lds.write(wave, f"hist{(pas + 1) % 3}", t, 0)
        c = np.array([[lds.read(wave, hc, 255 - 4 * l - j) for j in range(4)] for l in range(LANES)])
        sums = c.sum(axis=1)
        incl = np.cumsum(sums)
        excl = incl - sums
        found = np.zeros(LANES, bool)
        dsel = np.zeros(LANES, np.int64)
        abv = np.zeros(LANES, np.int64)
        for l in range(LANES):
            cum = excl[l]
            for j in range(4):
                if not found[l] and cum + c[l, j] >= remaining:
                    found[l], dsel[l], abv[l] = True, 255 - 4 * l - j, cum
                cum += c[l, j]
        found &= excl < remaining
        fl = int(np.nonzero(found)[0][0]) if found.any() else 0
        digit, above = int(dsel[fl]) & 255, int(abv[fl])
        prefix |= digit << shift
        mask |= 255 << shift
        remaining = remaining - above if remaining > above else 0
    T, take_eq = prefix, remaining
    shared.setdefault("T", set()).add((T, take_eq))
    per = (cand + NT - 1) // NT
    lo = np.minimum(cand, tid * per)
    hi = np.minimum(cand, lo + per)
    keys = shared["keys"]
    gt = np.zeros(LANES, np.int64)
    eq = np.zeros(LANES, np.int64)
    for l in range(LANES):
        for i in range(lo[l], hi[l]):
            lds.read(wave, "z", i)
            gt[l] += keys[i] > T
            eq[l] += keys[i] == T
    packed = (gt << 16) | eq
    incl = np.cumsum(packed)
    lds.write(wave, "wsum", wave, int(incl[-1]))
    yield
    before = sum(v for w, v in ((w, lds.read(wave, "wsum", w)) for w in range(WAVES)) if w < wave)
    excl = before + incl - packed
    eq_before = excl & 0xFFFF
    for l in range(LANES):
        taken_before = min(int(eq_before[l]), take_eq)
        p = (int(excl[l]) >> 16) + taken_before
        take = min(int(eq[l]), take_eq - taken_before)
        taken = 0
        for i in range(lo[l], hi[l]):
            keep = keys[i] > T
            if keys[i] == T and taken < take:
                keep, taken = True, taken + 1
            ok = keep and p < k
            if ok:
                assert 0 <= p < B
                lds.write(wave, "ks", p, i)
            lds.write(wave, "pos", i, p if ok else -1)
            p += keep
    for t in tid[tid < W]:
        lds.write(wave, "ks", k + t, cand + t)
        lds.write(wave, "pos", cand + t, k + t)
    yield


def run_model(z, N, B, W, rng, clear_late=False):
    keys = order_key(np.asarray(z, np.float32))
    lds = Lds(dict(z=np.arange(N), hist0=np.full(256, 99), hist1=np.full(256, 99),
                   hist2=np.full(256, 99), wsum=np.zeros(WAVES), ks=np.full(B, -7),
                   pos=np.full(N, -9)))
    shared = dict(keys=keys)
    progs = [wave_program(w, N, B, W, lds, shared, clear_late) for w in range(WAVES)]
    live = list(range(WAVES))
    while live:
        done = []
        for w in rng.permutation(live):          # the waves of one epoch, in a random order
            try:
                next(progs[w])
            except StopIteration:
                done.append(w)
        live = [w for w in live if w not in done]
        lds.epoch += 1
    assert len(shared["T"]) == 1, "waves disagree on the threshold"
    return lds.mem["ks"], lds.mem["pos"], lds.conflicts()


CASES = [
    # (N, B, W, kind)
    (1152, 1024, 8, "normal"), (2176, 2048, 8, "normal"), (70, 40, 8, "normal"),
    (9, 8, 1, "normal"), (130, 9, 8, "ties"), (300, 120, 1, "ties"), (1153, 1152, 8, "normal"),
    (700, 512, 8, "zeros"), (2176, 2048, 8, "ties"), (600, 300, 8, "constant"),
    (1200, 640, 8, "normal"), (520, 519, 1, "ties"), (127, 100, 30, "normal"),
]


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}-B{c[1]}-W{c[2]}-{c[3]}" for c in CASES])
def test_lean_select_model(case, seed):
    N, B, W, kind = case
    rng = np.random.default_rng(1000 * seed + N)
    if kind == "normal":
        z = (-0.9 * rng.uniform(0, 1, N) + 0.1 * rng.uniform(0, 0.01, N)).astype(np.float32)
    elif kind == "ties":
        z = rng.integers(-3, 3, N).astype(np.float32) * np.float32(0.25)
    elif kind == "zeros":
        z = np.where(rng.uniform(size=N) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        z[rng.integers(0, N, 20)] = -0.5
    else:
        z = np.full(N, -0.3, dtype=np.float32)
    ks, pos, bad = run_model(z, N, B, W, rng)
    assert not bad, f"LDS conflicts between waves within an epoch: {bad[:5]}"
    ref = orc.select(z.astype(np.float64), N, B, W)
    assert np.array_equal(ks, ref)
    expect = np.full(N, -1)
    expect[ref] = np.arange(B)
    assert np.array_equal(pos, expect)


def test_model_reports_a_late_clear():
    """With the next pass's histogram cleared after the barrier, waves clear
    it in the epoch where others add to it: the check reports the race."""
    rng = np.random.default_rng(5)
    z = (-0.9 * rng.uniform(0, 1, 1152)).astype(np.float32)
    _, _, bad = run_model(z, 1152, 1024, 8, rng, clear_late=True)
    assert bad


def test_race_check_catches_a_missing_barrier():
    """The same model with the clear of the next pass's histogram moved after
    the barrier (into the epoch where other waves already add to it) must
    report conflicts: the check is able to see such a race."""
    lds = Lds(dict(h=np.zeros(4)))
    lds.epoch = 3
    lds.write(0, "h", 1, 0)          # wave 0 clears ...
    lds.atomic_add(5, "h", 1, 1)     # ... while wave 5 adds in the same epoch
    assert lds.conflicts()
    lds2 = Lds(dict(h=np.zeros(4)))
    lds2.atomic_add(0, "h", 1, 1)
    lds2.atomic_add(5, "h", 1, 1)
    assert not lds2.conflicts()
