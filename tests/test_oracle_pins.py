"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("seed", range(12))
def test_bruteforce(seed):
    pins.check_bruteforce(seed)


@pytest.mark.parametrize("seed", range(12))
def test_select_ties(seed):
    pins.check_select_ties(seed)


@pytest.mark.parametrize("seed", range(4))
def test_lambda_extremes(seed):
    pins.check_lambda_one(seed)
    pins.check_lambda_zero(seed)


@pytest.mark.parametrize("seed", range(4))
def test_redundancy_closed_forms(seed):
    pins.check_duplicates(seed)
    pins.check_orthogonal(seed)
    pins.check_scale_invariance(seed)


@pytest.mark.parametrize("seed", range(4))
def test_importance_closed_forms(seed):
    pins.check_zero_queries(seed)
    pins.check_softmax_rows(seed)
    pins.check_identical_heads(seed)
    pins.check_logit_scale(seed)


def test_hand_example():
    pins.check_hand_example()


@pytest.mark.parametrize("seed", range(6))
def test_structure(seed):
    pins.check_structure(seed)


@pytest.mark.parametrize("seed", range(3))
def test_paged_closed_form(seed):
    pins.check_paged(seed)


@pytest.mark.parametrize("seed", range(4))
def test_redundancy_rows(seed):
    pins.check_redundancy_rows(seed)


@pytest.mark.parametrize("seed", range(8))
def test_bruteforce_variants(seed):
    pins.check_bruteforce_variants(seed)


@pytest.mark.parametrize("seed", range(4))
def test_variant_closed_forms(seed):
    pins.check_symmetric_closed_forms(seed)
    pins.check_unmasked_closed_forms(seed)
    pins.check_pooling_closed_forms(seed)


@pytest.mark.parametrize("seed", range(6))
def test_shared_selection(seed):
    pins.check_shared(seed)


@pytest.mark.parametrize("seed", range(4))
def test_paged_shared_selection(seed):
    pins.check_paged_shared(seed)


def test_budget_not_above_window_is_invalid():
    import numpy as np
    from oracle import rkv_oracle as orc
    with pytest.raises(ValueError):
        orc.select(np.zeros(10), 10, 4, 4)
