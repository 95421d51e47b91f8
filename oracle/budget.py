"""Adaptive verification budget — oracle side (test infrastructure).

Follows the budget as the pages describe it:

* FOS blog "추측 디코딩과 vLLM 적응형 검증", section "적응형 검증 > 동작"
  (Adaptive verification > How it works), steps 1-3: every draft slot is
  scored by its survival probability (the running product of per-position
  acceptance estimates), slots are ranked across the whole batch, and a cost
  model chosen at server start decides how many to keep by maximising
  expected accepted tokens over expected step time.
* agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive Verification)",
  section "DSpark 신뢰도 스케줄링 메커니즘" (Global Top-B Selection, Budget
  Calculation) and section "기술적 구현 및 CUDA Graphs" (Cost Modeling,
  CUDA Graph Padding): the numerator is one bonus token per sampling request
  plus the survivals of the B best slots; the denominator is the profiled cost
  of a step with T non-draft tokens plus B draft tokens; the cost curve is
  forced monotone and padded to the captured-graph staircase.

Readings where the pages are silent (each listed in the design notes):
confidences outside [0, 1] are clamped and NaN counts as 0; ties in the
ranking go to the lower request index and then the lower position; ties in
the objective go to the smallest B; survival products are taken in fp32 and
budget sums exactly in units of 2**-40.
"""

import math
from fractions import Fraction  # noqa: F401  (used by callers that check exactness)

import numpy as np

# Device error bits raised by budget selection (same values as the library's).
DEV_BAD_DRAFT_LEN = 8
DEV_BAD_COST = 16

FIXED_SHIFT = 40


def clamp_confidence(c):
    """A per-position acceptance estimate as a probability in fp32.

    The FOS page (section "동작", step 1) treats the estimate as the chance
    that this position is accepted given the earlier ones, i.e. a
    probability.  NaN, negative values and -0 become +0; values above 1
    become 1.
    """
    c = np.float32(c)
    if np.isnan(c) or c <= 0:  # a probability carries no sign: -0 becomes +0 too
        return np.float32(0.0)
    if c > 1:
        return np.float32(1.0)
    return c


def survival(conf, draft_len, k_max):
    """Survival s[r, j-1] of draft position j = 1..K_r of request r.

    FOS blog, section "동작", step 1: the score of a position is the
    probability that every position up to it is accepted — the product of the
    request's per-position acceptance estimates from the front.  The product
    is accumulated left to right in fp32 (round to nearest even), starting
    from 1 for the non-draft position.  Entries past K_r are 0.  Also returns
    the effective draft lengths (out-of-range lengths clamped into [0, k_max])
    and the error bits.
    """
    conf = np.asarray(conf, dtype=np.float32).reshape(len(draft_len), k_max)
    n = len(draft_len)
    s = np.zeros((n, k_max), dtype=np.float32)
    lens = np.zeros(n, dtype=np.int64)
    err = 0
    for r in range(n):
        K = int(draft_len[r])
        if K < 0 or K > k_max:
            err |= DEV_BAD_DRAFT_LEN
            K = min(max(K, 0), k_max)
        lens[r] = K
        prev = np.float32(1.0)
        for j in range(K):
            prev = np.float32(prev * clamp_confidence(conf[r, j]))
            s[r, j] = prev
    return s, lens, err


def cost_table_prepare(raw, granule, out_len):
    """Cost per step token count t = 0..out_len-1 from a raw profiled table.

    agentlens page, section "기술적 구현 및 CUDA Graphs", item Cost Modeling:
    the profiled cost curve is forced to be monotone non-decreasing (reading:
    the running maximum from small t upward).  Item CUDA Graph Padding: a batch
    pays for the next captured graph size, e.g. 121 tokens cost what 128 do
    (reading: sizes are multiples of ``granule``; granule 1 means no padding).
    So cost[t] = max(raw[0..ceil_g(t)]).  Raw entries must be finite and > 0.
    """
    raw = np.asarray(raw, dtype=np.float32)
    if granule < 1 or out_len < 1:
        raise ValueError("granule and out_len must be >= 1")
    need = ((out_len - 1 + granule - 1) // granule) * granule + 1
    if len(raw) < need:
        raise ValueError(f"raw table has {len(raw)} entries; padding needs {need}")
    if not np.all(np.isfinite(raw)) or np.any(raw <= 0):
        raise ValueError("raw costs must be finite and positive")
    running = np.zeros(len(raw), dtype=np.float32)
    m = raw[0]
    for t in range(len(raw)):
        if raw[t] > m:
            m = raw[t]
        running[t] = m
    out = np.zeros(out_len, dtype=np.float32)
    for t in range(out_len):
        padded = ((t + granule - 1) // granule) * granule
        out[t] = running[padded]
    return out


def rank_slots(s, lens):
    """All draft slots (r, j) in global order.

    FOS blog, section "동작", step 2: slots are taken from the whole batch in
    decreasing score, requests competing with each other.  Ties: lower request
    first, then lower position (with that rule the kept set of each request is
    a front prefix even when survivals tie, because survival never increases
    with position).
    """
    slots = [(r, j) for r in range(len(lens)) for j in range(int(lens[r]))]
    return sorted(slots, key=lambda rj: (-float(s[rj[0], rj[1]]), rj[0], rj[1]))


def fixed_point(sv):
    """floor(s * 2**40) for an fp32 survival s in [0, 1], as an exact integer."""
    return int(math.floor(float(sv) * (2.0 ** FIXED_SHIFT)))


def expected_tokens(n_bonus, sorted_survivals):
    """Expected emitted tokens when the given slots are verified, in reals.

    agentlens page, Budget Calculation: one bonus token per sampling request
    plus the survival of each verified slot.  For one request verifying its
    first k slots this is the FOS page's mean acceptance length
    1 + sum of the cumulative acceptance rates (section "평균 수락 길이").
    """
    return float(n_bonus) + float(sum(float(x) for x in sorted_survivals))


def budget_score(n_bonus, s_fixed, cost_value):
    """Objective of one candidate B in fp64: (n_bonus + S*2**-40) / cost.

    Non-finite or non-positive cost makes the candidate unusable (-inf).
    """
    c = float(cost_value)
    if not math.isfinite(c) or c <= 0:
        return -math.inf
    return (float(n_bonus) + float(s_fixed) * (2.0 ** -FIXED_SHIFT)) / c


def budget_select(conf, draft_len, k_max, cost, t_base, n_bonus):
    """Kept draft counts b_r and budget B for one step.

    FOS blog, section "동작", step 3, and agentlens page, Budget Calculation:
    B maximises (bonus tokens + survivals of the B best slots) divided by the
    cost of a step of t_base + B tokens; the smallest B wins ties.  b_r is the
    number of request r's slots among the first B in the global ranking
    (agentlens, Global Top-B Selection: a contiguous prefix per request).

    Returns dict(kept, budget, survival, dev_error, order, scores).
    """
    n = len(draft_len)
    s, lens, err = survival(conf, draft_len, k_max)
    order = rank_slots(s, lens)
    cost = np.asarray(cost, dtype=np.float32)
    if len(cost) < t_base + n * k_max + 1:
        raise ValueError("cost table shorter than t_base + n*k_max + 1")
    scores = []
    total = 0
    best_b = 0
    best = None
    for b in range(len(order) + 1):
        if b > 0:
            r, j = order[b - 1]
            total += fixed_point(s[r, j])
        cval = float(cost[t_base + b])
        if not math.isfinite(cval) or cval <= 0:
            err |= DEV_BAD_COST
        sc = budget_score(n_bonus, total, cval)
        scores.append(sc)
        if best is None or sc > best:
            best, best_b = sc, b
    kept = np.zeros(n, dtype=np.int32)
    for r, _j in order[:best_b]:
        kept[r] += 1
    return dict(kept=kept, budget=best_b, survival=s, dev_error=err,
                order=order, scores=scores, lens=lens)


def budget_allocate(conf, draft_len, k_max, budget):
    """Kept draft counts for a budget B sized elsewhere.

    agentlens page, section "DSpark 신뢰도 스케줄링 메커니즘", item Execution
    Pipeline: B is sized ahead of time from the previous step's confidences,
    and only the allocation of slots to requests runs with the current ones;
    the allocation is the same Global Top-B Selection (the B best slots of
    the global ranking, a contiguous prefix per request).  Reading: a B above
    the current number of slots keeps every slot, a negative B keeps none.

    Returns dict(kept, budget_used, survival, dev_error).
    """
    n = len(draft_len)
    s, lens, err = survival(conf, draft_len, k_max)
    order = rank_slots(s, lens)
    used = min(max(int(budget), 0), len(order))
    kept = np.zeros(n, dtype=np.int32)
    for r, _j in order[:used]:
        kept[r] += 1
    return dict(kept=kept, budget_used=used, survival=s, dev_error=err)
