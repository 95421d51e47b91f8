"""Pins of the oracle's uniform draft length (one K for the batch, chosen by
goodput).  Each test checks it against something other than itself: the FOS
truncated-k table, exact rational arithmetic, the adaptive budget it must
agree with or stay below, and the DSD page's claim about K and batch size."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def fos_conditional_rates():
    cum = load("fos_truncated_k_table.json")["cumulative_acceptance"]
    prev, rates = 1.0, []
    for c in cum:
        rates.append(c / prev)
        prev = c
    return np.array([rates], dtype=np.float32)


def test_fos_table_is_goodput_of_one_request_under_position_cost():
    """FOS "토큰 수를 늘리면 손해인 지점": tokens per computed position =
    AL(k) / (k + 1).  With one request, cost[t] = t (every computed position
    costs the same) and t_base = 1, the goodput of K is that column; the table
    shows it falls with k, so K* = 0 (compute-bound: drafting never pays)."""
    g = load("fos_truncated_k_table.json")
    conf = fos_conditional_rates()
    cost = np.arange(0, 1 + 7 + 1, dtype=np.float32)
    cost[0] = 1.0  # never consulted (t >= t_base = 1)
    res = oracle.uniform_k_select(conf, [7], 7, cost, 1, 1)
    for row in g["rows"]:
        assert res["scores"][row["k"]] == pytest.approx(row["tokens_per_computed_position"],
                                                        abs=0.006)
        assert res["scores"][row["k"]] * (row["k"] + 1) == pytest.approx(
            row["mean_acceptance_length"], abs=0.006)
    assert res["k"] == 0 and res["kept"].tolist() == [0]
    # memory-bound (flat cost): goodput = AL(k) grows with k, so every draft is taken
    flat = oracle.uniform_k_select(conf, [7], 7, np.ones(9, np.float32), 1, 1)
    assert flat["k"] == 7
    for row in g["rows"]:
        assert flat["scores"][row["k"]] == pytest.approx(row["mean_acceptance_length"], abs=0.006)


@pytest.mark.parametrize("seed", range(30))
def test_exact_rational_argmax(seed):
    """Dyadic confidences (multiples of 1/8) and integer costs make every
    survival and sum exact: the oracle's K equals the exact-rational argmax
    (smallest K on ties)."""
    rng = np.random.default_rng(seed)
    n, k = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    conf = (rng.integers(0, 9, (n, k)) / 8.0).astype(np.float32)
    dl = rng.integers(0, k + 1, n)
    t_base = n
    cost = (1 + np.floor(np.maximum(0, np.arange(t_base + n * k + 1) - rng.integers(0, 2 * n))
                         / rng.integers(1, 4))).astype(np.float32)
    res = oracle.uniform_k_select(conf, dl, k, cost, t_base, n)
    best, best_k = None, None
    for K in range(k + 1):
        num = Fraction(n)
        t = 0
        for r in range(n):
            s = Fraction(1)
            for j in range(min(K, int(dl[r]))):
                s *= Fraction(float(conf[r, j]))
                num += s
            t += min(K, int(dl[r]))
        val = num / Fraction(float(cost[t_base + t]))
        if best is None or val > best:
            best, best_k = val, K
    assert res["k"] == best_k
    assert res["kept"].tolist() == [min(best_k, int(x)) for x in dl]


@pytest.mark.parametrize("seed", range(20))
def test_single_request_equals_budget(seed):
    """With one request the adaptive budget's top-B slots are its first B
    positions (survival never rises along a request), so both choose the same
    count with the same scores."""
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(1, 9))
    conf = rng.uniform(0, 1, (1, k)).astype(np.float32)
    cost = np.maximum.accumulate(rng.uniform(0.5, 2.0, 1 + k + 1)).astype(np.float32)
    u = oracle.uniform_k_select(conf, [k], k, cost, 1, 1)
    b = oracle.budget_select(conf, [k], k, cost, 1, 1)
    assert u["k"] == b["budget"]
    assert u["scores"] == b["scores"]


@pytest.mark.parametrize("seed", range(20))
def test_budget_score_bounds_uniform(seed):
    """Every uniform K verifies some T draft slots; the adaptive budget's best
    T slots carry at least as much survival (floor is monotone), so its score
    at B = T is at least the uniform score, and its optimum at least K*'s."""
    rng = np.random.default_rng(200 + seed)
    n, k = int(rng.integers(2, 20)), int(rng.integers(1, 8))
    conf = rng.uniform(0.2, 1.0, (n, k)).astype(np.float32)
    dl = rng.integers(0, k + 1, n)
    cost = np.maximum.accumulate(1 + rng.uniform(0, 1, n + n * k + 1).cumsum() / n).astype(np.float32)
    u = oracle.uniform_k_select(conf, dl, k, cost, n, n)
    b = oracle.budget_select(conf, dl, k, cost, n, n)
    for K in range(k + 1):
        assert b["scores"][u["tokens"][K]] >= u["scores"][K]
    assert max(b["scores"]) >= max(u["scores"])


def test_k_falls_as_the_batch_reaches_the_compute_bound():
    """DSD page, section "동적 추측 디코딩(DSD)의 핵심 아이디어": K grows while
    the step is memory-bound and shrinks once it is compute-bound.  With the
    same acceptance per request and a cost flat up to 256 tokens then
    proportional, K* never rises with the batch size; it is the largest K for
    a small batch and 0 for a large one."""
    k = 8
    ks = []
    for n in [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512]:
        conf = np.full((n, k), 0.8, dtype=np.float32)
        t = np.arange(n + n * k + 1, dtype=np.float32)
        cost = np.maximum(1.0, t / 256.0).astype(np.float32)
        ks.append(oracle.uniform_k_select(conf, [k] * n, k, cost, n, n)["k"])
    assert all(a >= b for a, b in zip(ks, ks[1:])), ks
    assert ks[0] == k and ks[-1] == 0


def test_bad_lengths_and_costs_are_reported():
    conf = np.full((2, 3), 0.5, dtype=np.float32)
    cost = np.ones(2 + 6 + 1, dtype=np.float32)
    cost[2 + 1] = np.nan  # consulted at K = 1 (one token: the second length clamps to 0)
    res = oracle.uniform_k_select(conf, [5, -1], 3, cost, 2, 2)
    assert res["dev_error"] == oracle.DEV_BAD_DRAFT_LEN | oracle.DEV_BAD_COST
    assert res["scores"][1] == -np.inf
    assert res["kept"].tolist() == [res["k"], 0]
