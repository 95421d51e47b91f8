"""Draft-row features for acceptance prediction — oracle side (test infrastructure).

FOS blog "추측 디코딩과 vLLM 적응형 검증", section "켜는 방법과 제약" (the
table of where the per-position acceptance estimates come from): a drafter
without a confidence head gets its estimates from a small logistic model fed
with the draft's logits.  The features computed here summarise a draft row's
distribution — its largest probability and its entropy — from the row that
the verify step streams anyway.

Readings where the page leaves the step open (each listed in the design
notes):

* The distribution is the one the verify step uses for q: softmax(z / tau) at
  the verify temperature.
* Entropy is in bits, H = -sum_x q_x log2 q_x, with 0 log 0 = 0 (ids of
  logit -inf carry no probability and add nothing).
* The largest probability is max_x q_x.
* A row holding NaN or +inf, or only -inf, has no features (the verify step
  reports it as a fault).
"""

import numpy as np


def draft_features(z, tau):
    """(entropy in bits, largest probability) of softmax(z / tau), in fp64."""
    y = np.asarray(z, dtype=np.float64)
    if np.isnan(y).any() or np.isposinf(y).any() or np.isneginf(y).all():
        raise ValueError("row holds NaN or +inf, or only -inf")
    y = y / float(tau)
    e = np.exp(y - y.max())
    q = e / e.sum()
    pos = q[q > 0]
    entropy = float(-(pos * np.log2(pos)).sum()) + 0.0  # no -0
    return entropy, float(q.max())
