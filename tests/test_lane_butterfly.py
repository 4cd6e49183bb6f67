"""CPU model of the step-level column-max publish of the register-resident
kernels (publish_step in decode_kv_cache_03_amd/csrc/rkv_resident.hpp).

A wave holds, per lane, the max over its four accumulator rows for eight
(column block, column half) values; column cb*32 + cs*16 + l%16 of lane l.
The device reduces them over the four 16-lane quarters with lane swaps and
stores columns l and 64 + l from lane l. The model gives the gfx950 swaps
the meaning the kernels' pair16/pair32 helpers rely on: swapping register a
with register b exchanges the odd 16-lane rows (upper 32-lane half) of a with
the even rows (lower half) of b, so a lane gets (lower lane's value, upper
lane's value) when a and b are the same register. The test checks that the
helpers' meaning holds in the model and that every stored column is the
max over the four quarters, on random values with ties, infinities and
signed zeros. A last test checks the lanes that hold a fragment's diagonal
in the row-norm MFMA layout.
"""
import numpy as np

LANES = 64


def swap(a, b, width):
    """v_permlane16_swap (width 16) / v_permlane32_swap (width 32) of
    registers a and b: returns the two registers after the swap."""
    ra, rb = a.copy(), b.copy()
    for l in range(LANES):
        if (l // width) % 2 == 0:      # lower lane of its pair: b takes a's upper lane
            rb[l] = a[l + width]
        else:                          # upper lane: a takes b's lower lane
            ra[l] = b[l - width]
    return ra, rb


def publish_step(cm):
    """cm[l, cb, cs] -> the 128 stored column maxima (dst[0..127])."""
    r = []
    for i in range(4):                 # 16-lane stage: values 2i, 2i+1 = cm[:, i, 0], cm[:, i, 1]
        s0, s1 = swap(cm[:, i, 0], cm[:, i, 1], 16)
        r.append(np.maximum(s0, s1))
    o = []
    for i in range(2):                 # 32-lane stage
        s0, s1 = swap(r[2 * i], r[2 * i + 1], 32)
        o.append(np.maximum(s0, s1))
    dst = np.empty(128)
    dst[:64] = o[0]                    # lane l stores column l ...
    dst[64:] = o[1]                    # ... and column 64 + l
    return dst


def test_helper_meaning():
    """pair16/pair32 (swap of a register with itself) give the lower lane's
    value first, as the kernels' butterflies assume."""
    x = np.arange(LANES, dtype=np.float64)
    for width in (16, 32):
        lo, hi = swap(x, x, width)
        for l in range(LANES):
            low = l - width if (l // width) % 2 else l
            assert lo[l] == x[low] and hi[l] == x[low + width]


def test_every_column_is_the_max_over_quarters():
    rng = np.random.default_rng(0)
    for trial in range(300):
        cm = rng.standard_normal((LANES, 4, 2))
        if trial % 3 == 1:              # ties and special values
            cm = np.round(cm)
            cm[rng.random(cm.shape) < 0.1] = -np.inf
            cm[rng.random(cm.shape) < 0.05] = -0.0
        dst = publish_step(cm)
        for c in range(128):
            cb, cs, c16 = c // 32, (c % 32) // 16, c % 16
            want = max(cm[16 * q + c16, cb, cs] for q in range(4))
            assert dst[c] == want, (trial, c)


def test_a_single_quarter_decides():
    """Only one quarter holds a finite value per column: it must arrive."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        cm = np.full((LANES, 4, 2), -np.inf)
        owner = rng.integers(0, 4, size=(16, 4, 2))
        vals = rng.standard_normal((16, 4, 2))
        for c16 in range(16):
            for cb in range(4):
                for cs in range(2):
                    cm[16 * owner[c16, cb, cs] + c16, cb, cs] = vals[c16, cb, cs]
        dst = publish_step(cm)
        for c in range(128):
            assert dst[c] == vals[c % 16, c // 32, (c % 32) // 16]


def test_row_norm_diagonal_lanes():
    """Row norms from a fragment's product with itself (row_norms): lane l
    holds C[4q + v][l % 16] (q = l / 16), so the lanes with (l % 16) / 4 == q
    hold diagonal element l % 16 in accumulator v = l % 4. Each of the 16
    rows is written by exactly one lane, from the right accumulator entry."""
    writers = {}
    for l in range(LANES):
        c, q = l % 16, l // 16
        if (c >> 2) == q:
            v = c & 3
            assert 4 * q + v == c            # the entry is C[c][c]
            writers.setdefault(c, []).append(l)
    assert sorted(writers) == list(range(16))
    assert all(len(w) == 1 for w in writers.values())
