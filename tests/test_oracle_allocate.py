"""Pins for the oracle's allocation of a budget sized elsewhere (the stale-
confidence pipeline: B from the previous step, slots from the current one).

What fixes the answers here is not the oracle's ranking code:
* exhaustive search with exact rationals: for every B, the kept allocation
  carries the largest total survival over all per-request prefix allocations
  of B slots (the B best slots of the batch);
* agreement with budget selection when B is the budget it picks;
* the edge readings: a B above the slot count keeps everything, B <= 0 keeps
  nothing, sum(kept) = min(max(B, 0), slots).
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def best_prefix_total(s, lens, B):
    """Largest exact sum of survivals over allocations b_r <= K_r with sum B."""
    best = None
    for alloc in itertools.product(*[range(int(K) + 1) for K in lens]):
        if sum(alloc) != B:
            continue
        tot = sum(Fraction(float(s[r, j])) for r in range(len(lens)) for j in range(alloc[r]))
        best = tot if best is None or tot > best else best
    return best


@pytest.mark.parametrize("seed", range(40))
def test_allocation_takes_the_b_best_slots(seed):
    rng = np.random.default_rng(500 + seed)
    n, k = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    conf, dl, _cost, _t, _nb = workloads.random_budget_case(rng, n, k, ties=seed % 2 == 0,
                                                            zeros=seed % 5 == 0)
    total = int(np.clip(dl, 0, k).sum())
    for B in range(-1, total + 2):
        res = oracle.budget_allocate(conf, dl, k, B)
        kept, s = res["kept"], res["survival"]
        used = min(max(B, 0), total)
        assert res["budget_used"] == used and int(kept.sum()) == used
        assert np.all(kept <= np.clip(dl, 0, k))
        got = sum(Fraction(float(s[r, j])) for r in range(n) for j in range(int(kept[r])))
        assert got == best_prefix_total(s, np.clip(dl, 0, k), used), (B, kept)


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_allocation_at_the_selected_budget_is_the_selection(name):
    w = workloads.make(name)
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    sel = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    res = oracle.budget_allocate(w.conf, w.draft_len, w.k_max, sel["budget"])
    np.testing.assert_array_equal(res["kept"], sel["kept"])
    assert res["dev_error"] == sel["dev_error"] & oracle.DEV_BAD_DRAFT_LEN


def test_stale_budget_from_the_previous_step():
    """The pipeline's shape: B from step t-1's confidences, slots from step t's."""
    rng = np.random.default_rng(9)
    n, k = 64, 7
    cost = np.maximum(1.0, np.arange(n * k + n + 1) / 256.0).astype(np.float32)
    dl = np.full(n, k, dtype=np.int32)
    prev = (rng.beta(8, 2, (n, 1)) ** np.arange(1, k + 1)).astype(np.float32)
    cur = (rng.beta(8, 2, (n, 1)) ** np.arange(1, k + 1)).astype(np.float32)
    B = oracle.budget_select(prev, dl, k, cost, n, n)["budget"]
    res = oracle.budget_allocate(cur, dl, k, B)
    assert int(res["kept"].sum()) == B
    # the current step's own choice may differ, its allocation at B may not
    np.testing.assert_array_equal(
        res["kept"], oracle.budget_allocate(cur, dl, k, B)["kept"])
    # top-B: no slot left out survives better than a kept one
    s, kept = res["survival"], res["kept"]
    inside = [s[r, j] for r in range(n) for j in range(int(kept[r]))]
    outside = [s[r, j] for r in range(n) for j in range(int(kept[r]), k)]
    assert min(inside) >= max(outside)
