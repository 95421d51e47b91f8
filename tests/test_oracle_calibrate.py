"""Pins of the oracle's acceptance statistics and logistic calibration: a
hand-derived case, the FOS per-position table, finite differences of the
log-loss, unbiasedness of the gradient at the generating parameters, and the
direction of an update."""

import json
import math
import os

import numpy as np
import pytest

import oracle.calibrate as cal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cu_from_kept(kept):
    return np.concatenate([[0], np.cumsum(np.asarray(kept) + 1)]).astype(np.int32)


def test_hand_case():
    # r0 keeps 3, accepts 1 (verifies 0 ok, 1 rejected); r1 keeps 2, accepts both;
    # r2 keeps 0 (bonus only); r3 faulted (-1) and counts for nothing
    kept = [3, 2, 0, 4]
    res = cal.accept_stats([1, 2, 0, -1], cu_from_kept(kept), 4)
    assert res["attempted"].tolist() == [2, 2, 0, 0]
    assert res["accepted_at"].tolist() == [2, 1, 0, 0]
    assert res["requests"] == 3 and res["emitted"] == 2 + 3 + 1
    # an accepted count above the kept count is not a verify result: skipped
    res = cal.accept_stats([1, 3, 0], cu_from_kept([3, 2, 0]), 4)
    assert res["attempted"].tolist() == [1, 1, 0, 0] and res["requests"] == 2


def test_fos_per_position_table():
    """FOS per-position table: the conditional column is accepted_j / attempted_j
    and the cumulative column is accepted_j / requests; their running product
    agrees, and the mean acceptance length is 1 + the sum of the cumulative
    column (section "평균 수락 길이": 1.93 at k = 7)."""
    g = json.load(open(os.path.join(GOLDEN, "fos_truncated_k_table.json")))
    cum = g["cumulative_acceptance"]
    n, k = 100000, 7
    # requests accepting at least j+1 drafts: n * cum[j]
    at_least = [n] + [round(n * c) for c in cum]
    L = []
    for j in range(k + 1):
        count = at_least[j] - (at_least[j + 1] if j < k else 0)
        L += [j] * count
    res = cal.accept_stats(np.array(L), cu_from_kept([k] * len(L)), k)
    cond = res["accepted_at"] / res["attempted"]
    prod = np.cumprod(cond)
    np.testing.assert_allclose(prod, np.array(cum), atol=1e-5)
    np.testing.assert_allclose(res["accepted_at"] / res["requests"], cum, atol=1e-5)
    assert res["emitted"] / res["requests"] == pytest.approx(1 + sum(cum), abs=1e-4)
    assert res["emitted"] / res["requests"] == pytest.approx(g["rows"][7]["mean_acceptance_length"],
                                                             abs=0.006)


def synthetic(rng, n, k, theta):
    """Draft features and outcomes drawn from the logistic model theta: a
    request stops at its first rejection (the verify rule)."""
    kept = rng.integers(0, k + 1, n)
    q = np.where(rng.uniform(size=(n, k)) < 0.05, 0.0, rng.uniform(0.01, 1.0, (n, k)))
    h = rng.uniform(0.0, 8.0, (n, k))
    m = rng.uniform(0.05, 1.0, (n, k))
    L = np.zeros(n, dtype=np.int64)
    for r in range(n):
        j = 0
        while j < kept[r]:
            z = (theta[j] + theta[k] * cal.feature(q[r, j]) + theta[k + 1] * h[r, j]
                 + theta[k + 2] * m[r, j])
            if rng.uniform() >= cal.sigmoid(z):
                break
            j += 1
        L[r] = j
    return q, h, m, L, cu_from_kept(kept)


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(3)
    k = 4
    theta = rng.normal(0, 0.3, k + 3)
    q, h, m, L, cu = synthetic(rng, 300, k, rng.normal(0, 0.3, k + 3))
    g, count = cal.gradient(theta, q, L, cu, k, h, m)
    assert count > 0
    eps = 1e-6
    for i in range(k + 3):
        tp, tm = theta.copy(), theta.copy()
        tp[i] += eps
        tm[i] -= eps
        fd = (cal.log_loss(tp, q, L, cu, k, h, m) - cal.log_loss(tm, q, L, cu, k, h, m)) / (2 * eps)
        assert g[i] == pytest.approx(fd, rel=1e-5, abs=1e-6), i


def test_gradient_is_unbiased_at_the_generating_parameters():
    """With outcomes drawn from theta*, the mean gradient at theta* is ~0 and
    clearly not ~0 at a shifted theta."""
    rng = np.random.default_rng(5)
    k = 3
    star = np.array([1.2, 0.4, -0.3, 0.25, -0.2, 0.8])
    q, h, m, L, cu = synthetic(rng, 40000, k, star)
    g, count = cal.gradient(star, q, L, cu, k, h, m)
    assert np.all(np.abs(g / count) < 0.012), g / count
    off = star + np.array([0.5, -0.5, 0.5, 0.1, 0.1, -0.3])
    g2, _ = cal.gradient(off, q, L, cu, k, h, m)
    assert np.max(np.abs(g2 / count)) > 0.03


def test_absent_features_read_as_zero():
    rng = np.random.default_rng(8)
    k = 3
    theta = rng.normal(0, 0.5, k + 3)
    q, h, m, L, cu = synthetic(rng, 200, k, theta)
    g0, c0 = cal.gradient(theta, q, L, cu, k)
    g1, c1 = cal.gradient(theta, q, L, cu, k, np.zeros_like(h), np.zeros_like(m))
    np.testing.assert_array_equal(g0, g1)
    assert c0 == c1 and g0[k + 1] == 0 and g0[k + 2] == 0


def test_update_moves_toward_the_outcomes():
    k = 2
    theta = np.zeros(k + 3)
    q = np.full((4, k), 0.5)
    all_acc, _ = cal.calibrate_update(theta, q, [2, 2, 2, 2], cu_from_kept([2] * 4), k, 1.0)
    all_rej, _ = cal.calibrate_update(theta, q, [0, 0, 0, 0], cu_from_kept([2] * 4), k, 1.0)
    assert all_acc[0] > 0 and all_acc[1] > 0
    assert all_rej[0] < 0 and all_rej[1] == 0  # position 1 never verified
    # x_1 = log2 0.5 = -1 < 0: accepting pushes beta_1 down, rejecting up
    assert all_acc[k] < 0 and all_rej[k] > 0
    # by hand, at theta = 0 every prediction is 1/2 and x = (-1, 0, 0):
    # all accepted — 8 verified positions, each with error -1/2, so
    # grad = (-2, -2, 4, 0, 0) and the step subtracts grad / 8;
    # all rejected — 4 verified positions (position 0), error +1/2, so
    # grad = (2, 0, -2, 0, 0) and the step subtracts grad / 4
    np.testing.assert_array_equal(all_acc, [0.25, 0.25, -0.5, 0.0, 0.0])
    np.testing.assert_array_equal(all_rej, [-0.5, 0.0, 0.5, 0.0, 0.0])
    half, _ = cal.calibrate_update(theta, q, [2, 2, 2, 2], cu_from_kept([2] * 4), k, 0.5)
    np.testing.assert_array_equal(half, all_acc / 2)


def test_predict_and_features():
    assert cal.feature(0.0) == -64 and cal.feature(1.0) == 0 and cal.feature(0.25) == -2
    assert cal.feature(float("nan")) == -64 and cal.feature(2.0) == 0
    # a positive probability below 2**-64 sits at the floor too
    assert cal.feature(2.0 ** -100) == -64 and cal.feature(2.0 ** -64) == -64
    assert cal.feature(2.0 ** -63) == -63
    assert cal.entropy_feature(-1.0) == 0 and cal.entropy_feature(float("nan")) == 0
    assert cal.entropy_feature(3.5) == 3.5 and cal.entropy_feature(100.0) == 64
    assert cal.max_feature(-1.0) == 0 and cal.max_feature(float("nan")) == 0
    assert cal.max_feature(0.25) == 0.25 and cal.max_feature(1.5) == 1
    theta = np.array([0.0, math.log(3.0), 1.0, 0.5, -2.0])
    c = cal.predict(theta, np.array([[1.0, 0.5]]), 2)
    assert c[0, 0] == pytest.approx(0.5)
    assert c[0, 1] == pytest.approx(cal.sigmoid(math.log(3.0) - 1.0))
    c = cal.predict(theta, np.array([[1.0, 0.5]]), 2, np.array([[2.0, 4.0]]),
                    np.array([[0.5, 0.25]]))
    assert c[0, 0] == pytest.approx(cal.sigmoid(0.5 * 2.0 - 2.0 * 0.5))
    assert c[0, 1] == pytest.approx(cal.sigmoid(math.log(3.0) - 1.0 + 0.5 * 4.0 - 2.0 * 0.25))
