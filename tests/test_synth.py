"""Input generators: bf16 rounding and the workload structure (no GPU)."""
import numpy as np
import pytest

from synth import (CONFIGS, bf16_round, dense_case_host, paged_case_host, segment_layout,
                   tiny_head_case)


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("seed", range(5))
def test_segment_layout(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = 1152
    src = segment_layout(rng, n, 0.40)
    cov = (src >= 0).mean()
    assert 0.40 <= cov <= 0.41 + 1e-9
    t = np.nonzero(src >= 0)[0]
    assert np.all(src[t] < t)
    # copied positions are fresh in the source stream is not required; only earlier


def test_tiny_case_shape():
    c = tiny_head_case(0)
    assert c.K.shape == (1, 96, 128) and c.Q.shape == (1, 4, 8, 128)
    assert len(c.meta["dup_positions"]) == 29
    assert np.all(c.meta["dup_sources"] < c.meta["dup_positions"])


def test_dense_host_exact_bf16():
    c = dense_case_host(1, batch=1, layers=1, kv_heads=2, gqa=4, n=300, budget=256, window=8,
                        lam=0.1)
    assert np.array_equal(bf16_round(c.K), c.K)
    assert 0.39 <= c.meta["coverage"] <= 0.42


def test_paged_host_layout():
    c = paged_case_host(0, [40, 100, 130], [0.5, 0.3, 0.4], kv_heads=2, gqa=2, window=4)
    used = c.page_table[c.page_table >= 0]
    allp = np.concatenate([used, c.free_list])
    assert sorted(allp.tolist()) == list(range(c.meta["pool"]))
    assert np.all(c.budget % 16 == 0)


def test_configs_present():
    assert sorted(CONFIGS) == [0, 1, 2, 3, 4]


def test_decode_stream_rows_are_counter_based():
    """Rows of a step depend only on (seed, unit, step); copy steps equal the
    source step's fresh key plus small noise."""
    import torch
    from synth.decode_gen import DecodeStream
    s = DecodeStream(3, batch=2, layers=2, kv_heads=2, gqa=2, steps=300, coverage=0.4,
                     max_back=64, dtype="f32", device="cpu")
    k1, v1, q1 = s.rows(150)
    k2, v2, q2 = s.rows(150)
    assert torch.equal(k1, k2) and torch.equal(v1, v2) and torch.equal(q1, q2)
    assert k1.shape == (8, 128) and q1.shape == (8, 2, 128)
    lay = s.layouts
    assert 0.39 <= (lay >= 0).mean() <= 0.41
    seq, t = np.argwhere(lay >= 0)[0]
    src = lay[seq, t]
    assert 0 < t - src <= 64
    kt = s.rows(int(t))[0][seq * 4:(seq + 1) * 4]
    ks = s.rows(int(src))[0][seq * 4:(seq + 1) * 4]
    diff = (kt - ks).numpy()
    assert 0.005 < diff.std() < 0.05                       # sigma = 0.02 noise
    fresh = np.argwhere(lay[seq] < 0)[:, 0]
    a, b = s.rows(int(fresh[0]))[0], s.rows(int(fresh[1]))[0]
    assert abs(float(a.std()) - 1.0) < 0.1 and abs(float(torch.corrcoef(torch.stack([a.flatten(), b.flatten()]))[0, 1])) < 0.1
