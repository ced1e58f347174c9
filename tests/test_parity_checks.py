"""CPU checks of the acceptance checks themselves: a check that passes a wrong result proves
nothing, so each rule is run here on planted inputs it must accept and inputs it must reject."""
import numpy as np
import pytest
import torch

from tests.parity_util import (GAP, assert_close, bf16_rounding_interval, check_level,
                               lse_tolerance)


def _coarsest(scores):
    """A one-query coarsest level whose fp64 scores are `scores` (head_dim 1: q = 1, k = s)."""
    return np.ones((1, 1)), np.asarray(scores, dtype=np.float64)[:, None]


def test_tie_window_rejects_a_set_that_drops_the_best_candidate():
    # scores 10, 5, 5 (1 - 1e-6), K = 2: the oracle keeps {0, 1}; {1, 2} differs from it only
    # in a near tie at the K-th place but drops the clear winner 0
    q, k = _coarsest([10.0, 5.0, 5.0 * (1 - 1e-6)])
    with pytest.raises(AssertionError, match="left out"):
        check_level([[1, 2]], q, k, None, 2, "planted")


def test_tie_window_accepts_a_near_tie_swap():
    q, k = _coarsest([10.0, 5.0, 5.0 * (1 - 1e-6)])
    assert check_level([[0, 2]], q, k, None, 2, "swap") == 1
    assert check_level([[0, 1]], q, k, None, 2, "same") == 0


@pytest.mark.parametrize("row", [[0, 2], [1, 2]])
def test_tie_window_rejects_a_swap_outside_the_window(row):
    q, k = _coarsest([10.0, 5.0, 5.0 * (1 - 3 * GAP)])
    with pytest.raises(AssertionError):
        check_level([row], q, k, None, 2, "wide")


def test_tie_window_rejects_malformed_rows():
    q, k = _coarsest([3.0, 2.0, 2.0, 1.0])
    with pytest.raises(AssertionError, match="ascending"):
        check_level([[2, 0]], q, k, None, 2)
    with pytest.raises(AssertionError, match="ascending"):
        check_level([[1, 1]], q, k, None, 2)


def test_tie_window_on_a_finer_level_checks_candidates():
    # level below the coarsest: query 0 ranks the 16 children of its parent's single pick 1
    rng = np.random.default_rng(0)
    q = rng.standard_normal((16, 4))
    kl = rng.standard_normal((48, 4))
    parent = np.array([[1]])
    s = kl[16:32] @ q[0]
    best = 16 + np.argsort(-s, kind="stable")[:2]
    rows = np.tile(np.sort(best), (16, 1))
    from oracle import llsa_oracle as orc
    want = orc.select_level(q, kl, parent, 16, 2)
    rows[1:] = want[1:]
    assert check_level(rows, q, kl, parent, 2) == 0
    bad = rows.copy()
    bad[0] = [0, 16]   # id 0 is not a child of block 1
    with pytest.raises(AssertionError, match="outside"):
        check_level(bad, q, kl, parent, 2)


def test_bf16_rounding_interval_matches_round_to_nearest_even():
    rng = np.random.default_rng(1)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 30,
                          np.float32([0.0, -0.0, 1.0, -1.0, 2.0 ** -130, 65504.0, 2.0, 0.5])])
    xb = torch.from_numpy(x32).to(torch.bfloat16)
    x = xb.double().numpy()
    lo, hi = bf16_rounding_interval(x)
    assert np.all(lo <= x) and np.all(x <= hi)
    # points just inside round to x, points just outside do not (checked in fp64 -> fp32 ->
    # bf16, away from the fp32 rounding of the endpoints)
    for ends, inward in ((lo, 1), (hi, -1)):
        gap = np.abs(hi - lo)
        inside = (ends + inward * 1e-3 * gap).astype(np.float32)
        outside = (ends - inward * 1e-3 * gap).astype(np.float32)
        back_in = torch.from_numpy(inside).to(torch.bfloat16).double().numpy()
        back_out = torch.from_numpy(outside).to(torch.bfloat16).double().numpy()
        nz = x != 0
        assert np.array_equal(back_in[nz], x[nz])
        assert not np.any(back_out[nz] == x[nz])


def test_bf16_rounding_interval_rejects_non_bf16_values():
    with pytest.raises(ValueError):
        bf16_rounding_interval(np.array([1.0 + 2.0 ** -20]))


def test_assert_close_uses_the_exact_interval_not_a_relative_slack():
    # at |ref| ~ 30 a bf16 half ulp is 2^-4 = 0.0625; the former 2^-8 |ref| slack was 0.117
    ref = np.array([30.0, -30.0, 0.25])
    tol = 2e-2
    x = torch.tensor(ref).to(torch.bfloat16)
    assert_close(x, ref, torch.bfloat16, "exact")
    # the stored number 30.125 takes (30.0625, 30.1875): its distance to 30 is 0.0625 > tol
    far = torch.tensor([30.125, -30.0, 0.25]).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        assert_close(far, ref, torch.bfloat16, "one ulp off")
    # a reference 0.07 from the stored 30.0 (i.e. 0.0075 beyond its interval) passes; one
    # 0.09 away (0.0275 beyond) does not
    assert_close(x, ref + np.array([0.07, 0.0, 0.0]), torch.bfloat16, "inside bound")
    with pytest.raises(AssertionError):
        assert_close(x, ref + np.array([0.09, 0.0, 0.0]), torch.bfloat16, "beyond bound")
    # fp32 outputs get no interval
    y = torch.tensor([1.0, 2.0], dtype=torch.float32)
    with pytest.raises(AssertionError):
        assert_close(y, np.array([1.0, 2.0 + 3e-2]), torch.bfloat16, "fp32 output",
                     tol_abs=tol)
    assert tol > 0


def test_assert_close_mean_rel():
    ref = np.linspace(1.0, 2.0, 1000)
    x = torch.tensor(ref * (1 + 8e-3)).to(torch.float32)
    with pytest.raises(AssertionError, match="mean-rel"):
        assert_close(x, ref, torch.bfloat16, "mean-rel", tol_abs=1.0)


def test_lse_tolerance_bounds():
    q = np.full((4, 64), 2.0)
    k = np.full((8, 64), 3.0)
    assert lse_tolerance(q, k, torch.float32) == 1e-4
    plain = lse_tolerance(q, k, torch.bfloat16)
    coarse = lse_tolerance(q, k, torch.bfloat16, levels=3)
    assert 1e-5 < plain < coarse < 2e-2
    # ||q||_1 = 128, max|k| = 3, scale 1/8: 48 (64 2^-24) + 1e-5
    assert plain == pytest.approx(1e-5 + 48 * 64 * 2.0 ** -24)
