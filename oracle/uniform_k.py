"""One draft length for the whole batch — oracle side (test infrastructure).

"Hardware-Aware Dynamic Speculative Decoding (DSD), feat. Cohere"
(PyTorch-KR forum), section "동적 추측 디코딩(DSD)의 핵심 아이디어": instead of
a fixed K, the number of draft tokens is chosen from how the model and the
hardware interact — more drafts while the step is bound by memory bandwidth,
fewer once it is bound by compute — by maximising goodput = AL / ITL, the
acceptance length over the inter-token latency.

Readings where the page leaves the step open (each listed in the design
notes):

* AL(K) comes from the same per-position acceptance estimates the adaptive
  budget uses: a request drafting K tokens emits on average 1 + the sum of its
  first K survivals (FOS blog "추측 디코딩과 vLLM 적응형 검증", section
  "평균 수락 길이"); over the batch, n_bonus + sum_r sum_{j <= min(K, K_r)} s_rj.
  A request whose drafter wrote fewer than K drafts verifies what it has.
* ITL(K) is the shaped step cost at the step's token count,
  cost[t_base + sum_r min(K, K_r)] — the table the adaptive budget reads
  (agentlens "vLLM DSpark을 활용한 적응형 검증", Cost Modeling).
* Sums are exact in units of 2**-40 and the ratio is fp64, as for the budget;
  the smallest K wins ties.
"""

import math

import numpy as np

from .budget import DEV_BAD_COST, budget_score, fixed_point, survival


def uniform_k_select(conf, draft_len, k_max, cost, t_base, n_bonus):
    """K* = argmax over K in 0..k_max of goodput(K); kept[r] = min(K*, K_r).

    Returns dict(k, kept, scores (fp64, K = 0..k_max), tokens (draft tokens
    verified at each K), dev_error).
    """
    n = len(draft_len)
    s, lens, err = survival(conf, draft_len, k_max)
    cost = np.asarray(cost, dtype=np.float32)
    if len(cost) < t_base + n * k_max + 1:
        raise ValueError("cost table shorter than t_base + n*k_max + 1")
    scores, tokens = [], []
    best_k, best = 0, None
    for K in range(k_max + 1):
        total = 0  # sum of floor(s * 2**40) over the verified slots
        t = 0
        for r in range(n):
            m = min(K, int(lens[r]))
            t += m
            for j in range(m):
                total += fixed_point(s[r, j])
        cval = float(cost[t_base + t])
        if not math.isfinite(cval) or cval <= 0:
            err |= DEV_BAD_COST
        sc = budget_score(n_bonus, total, cval)
        scores.append(sc)
        tokens.append(t)
        if best is None or sc > best:
            best, best_k = sc, K
    kept = np.minimum(lens, best_k).astype(np.int32)
    return dict(k=best_k, kept=kept, scores=scores, tokens=tokens, dev_error=err)
