"""Full-vocabulary verification of kept rows — oracle side (test infrastructure).

What is computed, and where the pages say so:

* FOS blog "추측 디코딩과 vLLM 적응형 검증", section "추측 디코딩이란":
  the target scores k drafts in one pass, giving k+1 positions; drafts are
  compared from the front and accepted up to the first mismatch; at the
  mismatch the target's own token is emitted, so a step emits at least one
  token even if every draft fails.
* Same page, section "속도, 메모리, 정확도에 주는 영향", row 정확도
  (accuracy): with the original paper's rejection-sampling rule the output
  distribution equals the target model's.  The pages do not print the rule;
  the oracle uses the standard one from the papers the FOS page links
  (Leviathan et al. 2023; Chen et al. 2023): accept draft d at a position
  with probability min(1, p(d)/q(d)); on rejection draw from the normalised
  residual max(0, p - q).
* Same page, section "평균 수락 길이": the leading 1 of the mean acceptance
  length is the token the target picks itself — the bonus token after the
  last accepted draft, drawn from the target row at that position.
* Greedy mode: the target "picks the token itself" as its argmax; a draft is
  accepted iff it equals that argmax.

Readings where the pages are silent (also listed in the design notes):
p and q use the same temperature tau (softmax of z / tau); q(d) = 0 accepts iff
p(d) > 0; a residual of zero mass falls back to p; the token draw is the
inverse CDF over ascending token id with a strict '>' test against v * W, and
if rounding leaves no such id the last id of positive weight is taken; argmax
ties go to the lowest id; the Philox counter is (request, position, step).

Faults (device error bits, same values as the library's): inconsistent
row offsets, draft ids outside [0, V), and rows holding NaN or +inf or only
-inf; a faulty request emits -1 everywhere.
"""

import numpy as np

from .features import draft_features
from .philox import uniforms

STOCHASTIC = 0
GREEDY = 1

DEV_BAD_CU_ROWS = 1
DEV_BAD_TOKEN = 2
DEV_NONFINITE = 4


def row_is_faulty(z):
    """True if a logit row holds NaN or +inf, or only -inf (no probability mass)."""
    z = np.asarray(z, dtype=np.float64)
    return bool(np.isnan(z).any() or np.isposinf(z).any() or np.isneginf(z).all())


def row_probs(z, tau):
    """softmax(z / tau) in fp64 (max-shifted; -inf logits get probability 0)."""
    y = np.asarray(z, dtype=np.float64) / float(tau)
    y = y - y.max()
    e = np.exp(y)
    return e / e.sum()


def accept(u, p_d, q_d):
    """Accept the draft iff u < min(1, p(d)/q(d)); q(d) = 0 accepts iff p(d) > 0."""
    if q_d == 0.0:
        return p_d > 0.0
    return u < p_d / q_d


def residual_weights(p, q):
    """(weights, mass) of the residual max(0, p - q); zero mass falls back to p."""
    w = np.maximum(0.0, p - q)
    mass = float(w.sum())
    if mass == 0.0:
        return p.copy(), mass
    return w, mass


def inverse_cdf(w, v):
    """Smallest id x with C(x) > v * C(V-1), C the inclusive cumulative sum.

    If rounding leaves no such id, the last id with positive weight.
    """
    c = np.cumsum(w)
    t = v * c[-1]
    hit = np.nonzero(c > t)[0]
    if len(hit):
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def _argmax_first(z):
    z = np.asarray(z, dtype=np.float64)
    return int(np.argmax(z))


def verify_request(r, trows, drows, dtoks, b, vocab, mode, tau, seed, step,
                   forced_l=None, keep_weights=False):
    """Verify one request with b kept drafts.

    trows: the b+1 target logit rows (row j scores draft position j+1; row b
    gives the bonus).  drows: the b draft logit rows (stochastic only).
    dtoks: the draft ids.  forced_l: replay with the accepted length forced
    (drafts < forced_l accepted, forced_l rejected if < b); the result then
    lists every forced decision that disagrees with the natural one.

    Returns a dict with tokens, L, p_d, q_d, u, ratio, q_entropy, q_max
    (the draft-row features of positions 0..b-1), residual_mass, fault.
    """
    out = dict(tokens=[], L=-1, p_d=[], q_d=[], u=[], ratio=[], q_entropy=[], q_max=[],
               residual_mass=-1.0, fault=0, overridden=[], weights=None, v=None)
    for j in range(b):
        if not (0 <= int(dtoks[j]) < vocab):
            out["fault"] |= DEV_BAD_TOKEN
    rows_needed = list(trows[: b + 1]) + (list(drows[:b]) if mode == STOCHASTIC else [])
    if any(row_is_faulty(z) for z in rows_needed):
        out["fault"] |= DEV_NONFINITE
    if out["fault"]:
        return out

    if mode == GREEDY:
        argmaxes = [_argmax_first(trows[j]) for j in range(b + 1)]
        L = b
        for j in range(b):
            if int(dtoks[j]) != argmaxes[j]:
                L = j
                break
        if forced_l is not None:
            L = int(forced_l)
        out["L"] = L
        out["tokens"] = [int(d) for d in dtoks[:L]] + [argmaxes[L]]
        out["argmax"] = argmaxes
        return out

    p = [row_probs(trows[j], tau) for j in range(b + 1)]
    q = [row_probs(drows[j], tau) for j in range(b)]
    for j in range(b):
        h, m = draft_features(drows[j], tau)
        out["q_entropy"].append(h)
        out["q_max"].append(m)
    decisions = []
    for j in range(b):
        d = int(dtoks[j])
        u, _ = uniforms(seed, r, j, step)
        pd, qd = float(p[j][d]), float(q[j][d])
        out["p_d"].append(pd)
        out["q_d"].append(qd)
        out["u"].append(u)
        out["ratio"].append(np.inf if qd == 0.0 else pd / qd)
        decisions.append(accept(u, pd, qd))
    natural = b
    for j in range(b):
        if not decisions[j]:
            natural = j
            break
    L = natural if forced_l is None else int(forced_l)
    if forced_l is not None:
        for j in range(min(L + 1, b)):
            want = j < L
            if want != decisions[j]:
                out["overridden"].append((j, abs(out["u"][j] - out["ratio"][j])))
    if L < b:
        w, mass = residual_weights(p[L], q[L])
        out["residual_mass"] = mass
    else:
        w = p[b]
    _, v = uniforms(seed, r, L, step)
    tok = inverse_cdf(w, v)
    out["L"] = L
    out["tokens"] = [int(d) for d in dtoks[:L]] + [tok]
    out["v"] = v
    if keep_weights:
        out["weights"] = w
    return out


def verify(target, draft, draft_tokens, cu_rows, k_max, vocab, mode, temperature,
           seed=0, step=0, target_rows=None, forced=None, keep_weights=False):
    """Verify a packed batch.

    target: [rows, V] packed target logits (request r owns rows cu_rows[r] ..
    cu_rows[r+1]-1).  draft: [n*k_max, V] (or [n, k_max, V]) draft logits,
    row r*k_max + j for position j; None in greedy mode.  forced: optional
    {r: L} replays.  Returns dict(tokens [n, k_max+1], accepted [n], p_draft,
    q_draft, q_entropy, q_max [n, k_max] (stochastic, kept positions; -1
    elsewhere), residual_mass [n], dev_error, per_request).
    """
    cu_rows = np.asarray(cu_rows, dtype=np.int64)
    n = len(cu_rows) - 1
    target = np.asarray(target)
    rows_avail = target.shape[0] if target_rows is None else int(target_rows)
    if draft is not None:
        draft = np.asarray(draft)
        draft = draft.reshape(n * k_max, draft.shape[-1])
    draft_tokens = np.asarray(draft_tokens).reshape(n, k_max)
    tokens = np.full((n, k_max + 1), -1, dtype=np.int32)
    accepted = np.full(n, -1, dtype=np.int32)
    p_draft = np.full((n, k_max), -1.0)
    q_draft = np.full((n, k_max), -1.0)
    q_entropy = np.full((n, k_max), -1.0)
    q_max = np.full((n, k_max), -1.0)
    resid = np.full(n, -1.0)
    err = 0
    per_request = []
    for r in range(n):
        lo, hi = int(cu_rows[r]), int(cu_rows[r + 1])
        b = hi - lo - 1
        if lo < 0 or b < 0 or b > k_max or hi > rows_avail:
            err |= DEV_BAD_CU_ROWS
            per_request.append(None)
            continue
        trows = [target[lo + j, :vocab] for j in range(b + 1)]
        drows = [draft[r * k_max + j, :vocab] for j in range(b)] if mode == STOCHASTIC else []
        fl = None if forced is None else forced.get(r)
        res = verify_request(r, trows, drows, draft_tokens[r], b, vocab, mode,
                             temperature, seed, step, forced_l=fl,
                             keep_weights=keep_weights)
        per_request.append(res)
        if res["fault"]:
            err |= res["fault"]
            continue
        L = res["L"]
        accepted[r] = L
        tokens[r, : L + 1] = res["tokens"]
        if mode == STOCHASTIC:
            p_draft[r, :b] = res["p_d"]
            q_draft[r, :b] = res["q_d"]
            q_entropy[r, :b] = res["q_entropy"]
            q_max[r, :b] = res["q_max"]
            resid[r] = res["residual_mass"]
    return dict(tokens=tokens, accepted=accepted, p_draft=p_draft, q_draft=q_draft,
                q_entropy=q_entropy, q_max=q_max, residual_mass=resid, dev_error=err, per_request=per_request)
