"""Pins for the oracle's survival, cost shaping and budget selection (CPU only).

What fixes the answers here is not the oracle itself:
* the acceptance tables printed on the FOS page "추측 디코딩과 vLLM 적응형
  검증" (section "뒤 자리 수락률이 급하게 떨어지는 이유": per-position table and
  the 0.55**7 chain example; section "토큰 수를 늘리면 손해인 지점":
  truncated-k table), stored under tests/golden/ with their citations;
* the padding example on the agentlens page (121 tokens pay for 128);
* exhaustive search with exact rationals over every per-request allocation;
* invariants: survival never increases with position, the kept set is a
  front prefix of each request, shaped cost is monotone.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_survival_matches_per_position_table():
    g = load("fos_per_position_acceptance.json")
    cond = np.array([g["conditional"]], dtype=np.float32)
    s, lens, err = oracle.survival(cond, [7], 7)
    assert err == 0 and lens[0] == 7
    # cumulative = running product of the conditional column, to the printed 0.1 %
    np.testing.assert_allclose(s[0], g["cumulative"], atol=0.0006)
    # chain example: seven calls at 55 % each succeed together 1.5 % of the time
    s7, _, _ = oracle.survival(np.full((1, 7), 0.55, dtype=np.float32), [7], 7)
    assert round(float(s7[0, 6]) * 100, 1) == g["chain_example"]["all_seven_percent"]


def test_expected_tokens_and_cost_per_position_match_truncation_table():
    g = load("fos_truncated_k_table.json")
    cum = g["cumulative_acceptance"]
    for row in g["rows"]:
        k = row["k"]
        al = oracle.expected_tokens(1, cum[:k])
        assert round(al, 2) == row["mean_acceptance_length"]
        # a fully busy GPU: cost proportional to positions computed (t = 1 + k)
        fx = sum(oracle.fixed_point(np.float32(c)) for c in cum[:k])
        score = oracle.budget_score(1, fx, float(1 + k))
        assert round(score, 2) == row["tokens_per_computed_position"]
        if k:
            assert round(cum[k - 1], 3) == row["last_position_gain"]


def test_budget_extremes_follow_the_pages():
    g = load("fos_truncated_k_table.json")
    cum = np.array(g["cumulative_acceptance"], dtype=np.float64)
    cond = np.array([cum[0]] + list(cum[1:] / cum[:-1]), dtype=np.float32)[None, :]
    # compute-bound cost (t tokens cost t): no draft is worth its position
    res = oracle.budget_select(cond, [7], 7, np.arange(0, 9, dtype=np.float32) + 0.0, 1, 1)
    assert res["budget"] == 0 and res["kept"][0] == 0
    # idle GPU (flat cost): every draft is verified, like a fixed k
    res = oracle.budget_select(cond, [7], 7, np.ones(9, dtype=np.float32), 1, 1)
    assert res["budget"] == 7 and res["kept"][0] == 7


def test_cost_padding_example_and_monotone():
    raw = np.linspace(1.0, 3.0, 200).astype(np.float32)
    raw[50] = 10.0  # profiling noise spike
    out = oracle.cost_table_prepare(raw, 16, 130)
    # agentlens page, CUDA Graph Padding: a 121-token batch costs the 128-token graph
    assert out[121] == oracle.cost_table_prepare(raw, 1, 129)[128]
    assert out[121] == max(raw[:129])
    assert np.all(np.diff(out) >= 0)
    assert out[0] == raw[0] and out[1] == max(raw[:17])
    flat = oracle.cost_table_prepare(raw, 1, 200)
    np.testing.assert_array_equal(flat, np.maximum.accumulate(raw))
    with pytest.raises(ValueError):
        oracle.cost_table_prepare(raw, 16, 200)  # padding needs raw[208]
    bad = raw.copy()
    bad[3] = np.nan
    with pytest.raises(ValueError):
        oracle.cost_table_prepare(bad, 1, 10)
    with pytest.raises(ValueError):
        oracle.cost_table_prepare(-raw, 1, 10)


def test_clamp_and_survival_edge_cases():
    conf = np.array([[np.nan, 0.5, 2.0], [-1.0, np.inf, 0.25]], dtype=np.float32)
    s, lens, err = oracle.survival(conf, [3, 5], 3)
    assert err == oracle.DEV_BAD_DRAFT_LEN and list(lens) == [3, 3]
    np.testing.assert_array_equal(s, [[0, 0, 0], [0, 0, 0]])
    s, _, _ = oracle.survival(np.array([[0.5, 2.0, 0.5]], dtype=np.float32), [2], 3)
    np.testing.assert_array_equal(s, [[0.5, 0.5, 0.0]])
    # fp32 product, round to nearest even, denormals kept
    tiny = np.float32(2.0 ** -70)
    s, _, _ = oracle.survival(np.array([[tiny, tiny, 0.5]], dtype=np.float32), [3], 3)
    assert s[0, 1] == np.float32(2.0 ** -140) and s[0, 2] == np.float32(2.0 ** -141)



def test_confidence_sign_is_dropped():
    """A confidence is a probability (FOS "동작", step 1), so a survival is a
    number in [0, 1] and carries no sign: -0, negative values and NaNs of either
    sign clamp to +0 (bit pattern 0), and every survival is sign-free, so the
    fp32 bit patterns of survivals order like their values."""
    for c in (-0.0, -1e-45, -1.0, float("-nan"), float("nan")):
        assert oracle.clamp_confidence(c).view(np.uint32) == 0, c
    neg_nan = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)[0]
    conf = np.array([[0.5, -0.0, 0.5], [-0.0, 0.5, 0.5], [neg_nan, 1.0, 1.0]],
                    dtype=np.float32)
    s, _, _ = oracle.survival(conf, [3, 3, 3], 3)
    assert not np.signbit(s).any()
    np.testing.assert_array_equal(s.view(np.uint32),
                                  np.array([[0x3F000000, 0, 0], [0, 0, 0], [0, 0, 0]],
                                           dtype=np.uint32))
    assert oracle.clamp_confidence(np.float32(2.0 ** -149)) == np.float32(2.0 ** -149)

def round_binary32(x):
    """The binary32 value nearest to the rational x >= 0 (IEEE 754
    roundTiesToEven: 24-bit significands, subnormals below 2**-126), written
    from the definition with exact rationals."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    scaled = x / quantum
    n = scaled.numerator // scaled.denominator
    rest = scaled - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * quantum


def test_survival_rounds_every_product_to_fp32():
    """Each survival is the previous one times the next confidence, rounded to
    binary32 at every step (not the exact product rounded once): checked against
    exact rationals rounded by the IEEE definition, on chains where the two
    differ."""
    rng = np.random.default_rng(77)
    n, k = 400, 8
    conf = rng.uniform(0.0, 1.0, (n, k)).astype(np.float32)
    conf[::7] = (conf[::7] * np.float32(2.0 ** -40)).astype(np.float32)  # into subnormals
    s, _, _ = oracle.survival(conf, [k] * n, k)
    differs = 0
    for r in range(n):
        chained, exact = Fraction(1), Fraction(1)
        for j in range(k):
            c = Fraction(float(conf[r, j]))
            chained = round_binary32(chained * c)
            exact *= c
            assert Fraction(float(s[r, j])) == chained, (r, j)
            differs += round_binary32(exact) != chained
    assert differs > 50  # the test tells the two roundings apart


def test_ties_go_to_the_lower_request_then_position():
    """Equal survivals rank by request, then position (the kept sets stay
    front prefixes either way; the reading fixes which request keeps the slot)."""
    half = np.full((3, 2), 0.5, dtype=np.float32)  # survivals 0.5, 0.25 everywhere
    order = oracle.rank_slots(*oracle.survival(half, [2, 2, 2], 2)[:2])
    assert order == [(0, 0), (1, 0), (2, 0), (0, 1), (1, 1), (2, 1)]
    assert oracle.budget_allocate(half, [2, 2, 2], 2, 2)["kept"].tolist() == [1, 1, 0]
    assert oracle.budget_allocate(half, [2, 2, 2], 2, 4)["kept"].tolist() == [2, 1, 1]
    ones = np.ones((2, 2), dtype=np.float32)  # survival 1 at every slot
    assert oracle.budget_allocate(ones, [2, 2], 2, 1)["kept"].tolist() == [1, 0]
    assert oracle.budget_allocate(ones, [2, 2], 2, 3)["kept"].tolist() == [2, 1]


def test_fixed_point_is_the_floor():
    """Budget sums count survivals in whole units of 2**-40, rounding down."""
    f32 = np.float32
    assert oracle.fixed_point(f32(1.0)) == 2 ** 40
    assert oracle.fixed_point(f32(0.5 + 2.0 ** -24)) == 2 ** 39 + 2 ** 16
    assert oracle.fixed_point(f32(7 * 2.0 ** -42)) == 1   # 1.75 units
    assert oracle.fixed_point(f32(3 * 2.0 ** -42)) == 0   # 0.75 units
    assert oracle.fixed_point(f32(2 * 2.0 ** -42)) == 0   # 0.5 units
    assert oracle.fixed_point(f32(2.0 ** -149)) == 0
    assert oracle.fixed_point(f32(0.0)) == 0


def exhaustive_best(s, lens, cost, t_base, n_bonus):
    """Best allocation over every (b_r) in prod {0..K_r}, exact rationals."""
    n = len(lens)
    best_val, best_b = None, None
    for alloc in itertools.product(*[range(int(k) + 1) for k in lens]):
        b = sum(alloc)
        c = Fraction(float(cost[t_base + b]))
        num = Fraction(n_bonus) + sum(Fraction(float(s[r, j])) for r in range(n)
                                      for j in range(alloc[r]))
        val = num / c
        if best_val is None or val > best_val or (val == best_val and b < best_b):
            best_val, best_b = val, b
    return best_val, best_b


@pytest.mark.parametrize("seed", range(60))
def test_budget_matches_exhaustive_search_dyadic(seed):
    """Confidences in multiples of 1/8 make survivals (and their 2**-40 fixed
    point) exact, so the oracle's choice must be the exact optimum, with the
    smallest B among exact ties."""
    rng = np.random.default_rng(seed)
    n, k = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(
        rng, n, k, ties=True, zeros=seed % 3 == 0, flat_cost=seed % 10 == 0)
    cost = (np.round(cost * 64) / 64).astype(np.float32)
    res = oracle.budget_select(conf, dl, k, cost, t_base, n_bonus)
    best_val, best_b = exhaustive_best(res["survival"], res["lens"], cost, t_base, n_bonus)
    kept = res["kept"]
    got_num = Fraction(n_bonus) + sum(Fraction(float(res["survival"][r, j]))
                                      for r in range(n) for j in range(int(kept[r])))
    got_val = got_num / Fraction(float(cost[t_base + int(kept.sum())]))
    # fp64 scores can only blur exact ties below one rounding of the quotient
    assert got_val == best_val or abs(got_val - best_val) <= best_val * Fraction(1, 2**51)
    if got_val == best_val:
        assert int(kept.sum()) == best_b
    assert res["budget"] == int(kept.sum())


@pytest.mark.parametrize("seed", range(40))
def test_budget_near_optimal_random(seed):
    """Arbitrary fp32 survivals: the fixed-point objective may differ from the
    exact one by at most (number of slots) * 2**-40 in the numerator."""
    rng = np.random.default_rng(1000 + seed)
    n, k = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(rng, n, k)
    res = oracle.budget_select(conf, dl, k, cost, t_base, n_bonus)
    best_val, _ = exhaustive_best(res["survival"], res["lens"], cost, t_base, n_bonus)
    kept = res["kept"]
    num = Fraction(n_bonus) + sum(Fraction(float(res["survival"][r, j]))
                                  for r in range(n) for j in range(int(kept[r])))
    got = num / Fraction(float(cost[t_base + int(kept.sum())]))
    slack = Fraction(n * k + 1, 2**40) / Fraction(float(cost.min())) + best_val * Fraction(1, 2**50)
    assert got >= best_val - slack


@settings(max_examples=150, deadline=None, derandomize=True)
@given(st.integers(1, 12), st.integers(1, 8), st.integers(0, 2**31 - 1),
       st.booleans(), st.booleans())
def test_kept_set_is_prefix_closed_and_ranked(n, k, seed, ties, zeros):
    rng = np.random.default_rng(seed)
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(rng, n, k, ties=ties,
                                                                   zeros=zeros)
    res = oracle.budget_select(conf, dl, k, cost, t_base, n_bonus)
    s, kept, order, B = res["survival"], res["kept"], res["order"], res["budget"]
    # survival never increases with position
    for r in range(n):
        K = int(res["lens"][r])
        assert np.all(np.diff(s[r, :K]) <= 0)
        assert 0 <= kept[r] <= K
    # the first B ranked slots are exactly the front prefixes of length kept[r]
    chosen = set(order[:B])
    assert chosen == {(r, j) for r in range(n) for j in range(int(kept[r]))}
    # the ranking is by survival, descending
    vals = [float(s[r, j]) for r, j in order]
    assert all(a >= b for a, b in zip(vals, vals[1:]))
    # B is the first maximiser of the recorded scores
    sc = res["scores"]
    assert B == int(np.argmax(sc)) and sc[B] == max(sc)


def test_bad_cost_entries_are_flagged_and_skipped():
    conf = np.full((2, 2), 0.9, dtype=np.float32)
    cost = np.array([1.0, 1.0, 1.0, 1.0, 1.0], dtype=np.float32)
    cost[4] = np.nan
    res = oracle.budget_select(conf, [2, 2], 2, cost, 0, 2)
    assert res["dev_error"] & oracle.DEV_BAD_COST
    assert res["budget"] == 3
    cost = np.array([0.0] * 5, dtype=np.float32)
    res = oracle.budget_select(conf, [2, 2], 2, cost, 0, 2)
    assert res["budget"] == 0 and res["dev_error"] & oracle.DEV_BAD_COST
    assert all(math.isinf(x) for x in res["scores"])


def test_tiny_workload_budget():
    w = workloads.make("tiny")
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    res = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    best_val, best_b = exhaustive_best(res["survival"], res["lens"], cost, w.t_base, w.n_bonus)
    assert res["budget"] == best_b
