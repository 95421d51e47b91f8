"""Acceptance statistics and online confidence calibration — oracle side (test infrastructure).

FOS blog "추측 디코딩과 vLLM 적응형 검증":

* section "켜는 방법과 제약" (the table of where the per-position acceptance
  estimates come from): for model-based drafters without a confidence head,
  a small logistic model predicts acceptance from the draft's logits and is
  recalibrated during serving from the actual verification results;
* the measurement checklist (item 4: per-position acceptance rate and mean
  acceptance length) and section "평균 수락 길이" (acceptance length = one
  plus the accepted drafts of a verify step).

Readings where the page leaves the step open (each listed in the design
notes):

* A position j of request r is verified when every earlier position was
  accepted and j < b_r: positions 0 .. min(L_r, b_r - 1).  Positions below L_r
  were accepted, position L_r (when L_r < b_r) was rejected, later positions
  are unobserved.  Requests whose outcome is not a verify result (L_r = -1
  after a fault, or L_r, b_r outside 0 <= L_r <= b_r <= k_max) contribute
  nothing.
* The model estimates the conditional acceptance of position j — the
  quantity the budget multiplies into survivals — as
  c_j = sigmoid(alpha_j + beta_1 x_1 + beta_2 x_2 + beta_3 x_3) from three
  features of the draft's logits at that position: x_1 = log2 q(d_j) clamped
  to [-64, 0] (the draft's own probability of its token), x_2 = the entropy
  of the draft row in bits, clamped to [0, 64], and x_3 = its largest
  probability, clamped to [0, 1] (NaN, or a feature left out, reads as 0;
  for x_1 as -64).  theta = [alpha_0 .. alpha_{K-1}, beta_1, beta_2, beta_3].
* One calibration step is one plain gradient step on the mean log-loss over
  the verified positions of the batch: theta <- theta - lr * grad / N.
"""

import math

import numpy as np

X_MIN = -64.0
H_MAX = 64.0
N_FEAT = 3


def feature(q):
    """x_1 = log2 q(d), clamped to [-64, 0]; q <= 0 (or NaN) reads as the floor."""
    q = float(q)
    if not (q > 0):
        return X_MIN
    return min(0.0, max(X_MIN, math.log2(q)))


def entropy_feature(h):
    """x_2 = entropy in bits, clamped to [0, 64]; NaN or negative reads as 0."""
    h = float(h)
    return min(H_MAX, h) if h > 0 else 0.0


def max_feature(m):
    """x_3 = largest probability, clamped to [0, 1]; NaN or negative reads as 0."""
    m = float(m)
    return min(1.0, m) if m > 0 else 0.0


def features(q_draft, q_entropy, q_max, r, j):
    """(x_1, x_2, x_3) of request r, position j; absent inputs read as 0."""
    return (feature(q_draft[r, j]),
            0.0 if q_entropy is None else entropy_feature(q_entropy[r, j]),
            0.0 if q_max is None else max_feature(q_max[r, j]))


def verified_positions(accepted, cu_rows, k_max):
    """Per request: (counted, list of (j, y)) of the verified positions."""
    n = len(accepted)
    out = []
    for r in range(n):
        b = int(cu_rows[r + 1]) - int(cu_rows[r]) - 1
        L = int(accepted[r])
        counted = 0 <= L <= b <= k_max
        obs = []
        if counted:
            for j in range(min(L, b - 1) + 1 if b > 0 else 0):
                obs.append((j, 1 if j < L else 0))
        out.append((counted, L, obs))
    return out


def accept_stats(accepted, cu_rows, k_max):
    """Counters of one verify step.

    attempted[j]: requests that verified position j; accepted_at[j]: of those,
    the ones that accepted it (so accepted_at[j] / attempted[j] is the
    conditional acceptance of position j, the FOS per-position table's
    conditional column); requests: requests counted; emitted: their emitted
    tokens, sum (L_r + 1) — emitted / requests is the mean acceptance length.
    """
    attempted = np.zeros(k_max, dtype=np.int64)
    accepted_at = np.zeros(k_max, dtype=np.int64)
    requests = emitted = 0
    for counted, L, obs in verified_positions(accepted, cu_rows, k_max):
        if not counted:
            continue
        requests += 1
        emitted += L + 1
        for j, y in obs:
            attempted[j] += 1
            accepted_at[j] += y
    return dict(attempted=attempted, accepted_at=accepted_at, requests=requests, emitted=emitted)


def sigmoid(z):
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def _as2d(a, k_max):
    return None if a is None else np.asarray(a, dtype=np.float64).reshape(-1, k_max)


def _logit(theta, k_max, j, x):
    return float(theta[j]) + sum(float(theta[k_max + i]) * x[i] for i in range(N_FEAT))


def predict(theta, q_draft, k_max, q_entropy=None, q_max=None):
    """c[r, j] = sigmoid(alpha_j + beta . x(r, j))."""
    q, h, m = _as2d(q_draft, k_max), _as2d(q_entropy, k_max), _as2d(q_max, k_max)
    c = np.zeros(q.shape, dtype=np.float64)
    for r in range(q.shape[0]):
        for j in range(k_max):
            c[r, j] = sigmoid(_logit(theta, k_max, j, features(q, h, m, r, j)))
    return c


def gradient(theta, q_draft, accepted, cu_rows, k_max, q_entropy=None, q_max=None):
    """Sum over verified positions of d(log-loss)/d(theta), and their count."""
    q, h, m = _as2d(q_draft, k_max), _as2d(q_entropy, k_max), _as2d(q_max, k_max)
    g = np.zeros(k_max + N_FEAT, dtype=np.float64)
    count = 0
    for r, (_c, _L, obs) in enumerate(verified_positions(accepted, cu_rows, k_max)):
        for j, y in obs:
            x = features(q, h, m, r, j)
            err = sigmoid(_logit(theta, k_max, j, x)) - y
            g[j] += err
            for i in range(N_FEAT):
                g[k_max + i] += err * x[i]
            count += 1
    return g, count


def log_loss(theta, q_draft, accepted, cu_rows, k_max, q_entropy=None, q_max=None):
    """Sum over verified positions of -log P(outcome) (used by the pins)."""
    q, h, m = _as2d(q_draft, k_max), _as2d(q_entropy, k_max), _as2d(q_max, k_max)
    total = 0.0
    for r, (_c, _L, obs) in enumerate(verified_positions(accepted, cu_rows, k_max)):
        for j, y in obs:
            z = _logit(theta, k_max, j, features(q, h, m, r, j))
            # -log sigmoid(z) = log(1 + e^-z); -log(1 - sigmoid(z)) = log(1 + e^z)
            total += math.log1p(math.exp(-abs(z))) + max(0.0, -z if y else z)
    return total


def calibrate_update(theta, q_draft, accepted, cu_rows, k_max, lr, q_entropy=None, q_max=None):
    """One gradient step on the mean log-loss of the verified positions."""
    g, count = gradient(theta, q_draft, accepted, cu_rows, k_max, q_entropy, q_max)
    theta = np.asarray(theta, dtype=np.float64).copy()
    if count:
        theta -= lr * g / count
    return theta, count
