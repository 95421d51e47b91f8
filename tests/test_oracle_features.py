"""Pins of the oracle's draft-row features (entropy in bits and largest
probability of softmax(z / tau)): closed forms on uniform, k-point and
two-point rows, scipy's entropy and softmax on random rows, and invariants
(shift, temperature folding, the min-entropy and support bounds, entropy
rising with temperature)."""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle.features import draft_features

NEG = -np.inf


@pytest.mark.parametrize("V", [1, 2, 7, 32000])
@pytest.mark.parametrize("tau", [0.3, 1.0, 2.5])
def test_uniform_row(V, tau):
    h, m = draft_features(np.full(V, 1.75), tau)
    assert h == pytest.approx(math.log2(V), abs=1e-12)
    assert m == pytest.approx(1.0 / V, rel=1e-12)


@pytest.mark.parametrize("k", [1, 3, 64])
def test_k_equal_logits_among_masked_ids(k):
    rng = np.random.default_rng(k)
    z = np.full(1000, NEG)
    z[rng.choice(1000, k, replace=False)] = -3.0
    h, m = draft_features(z, 0.7)
    assert h == pytest.approx(math.log2(k), abs=1e-12)
    assert m == pytest.approx(1.0 / k, rel=1e-12)
    assert math.copysign(1.0, h) == 1.0  # a one-point row gives +0, not -0


@pytest.mark.parametrize("d,tau", [(0.0, 1.0), (1.0, 1.0), (3.0, 0.5), (-2.0, 2.0), (40.0, 1.0)])
def test_two_point_closed_form(d, tau):
    # q = (1 / (1 + e^{d/tau}), e^{d/tau} / (1 + e^{d/tau})): binary entropy
    p1 = 1.0 / (1.0 + math.exp(d / tau))
    p2 = 1.0 - p1
    want = sum(-p * math.log2(p) for p in (p1, p2) if p > 0)
    h, m = draft_features(np.array([0.0, d, NEG]), tau)
    assert h == pytest.approx(want, abs=1e-12)
    assert m == pytest.approx(max(p1, p2), rel=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_matches_scipy(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 5000))
    z = rng.normal(0, 3, V)
    z[rng.uniform(size=V) < 0.1] = NEG
    z[0] = 0.0
    tau = float(rng.uniform(0.2, 3.0))
    q = scipy.special.softmax(np.where(np.isinf(z), -np.inf, z / tau))
    h, m = draft_features(z, tau)
    assert h == pytest.approx(scipy.stats.entropy(q, base=2), rel=1e-10, abs=1e-12)
    assert m == pytest.approx(q.max(), rel=1e-12)


def test_invariants():
    rng = np.random.default_rng(11)
    z = rng.normal(0, 3, 4096)
    z[::17] = NEG
    finite = int(np.isfinite(z).sum())
    prev = -1.0
    for tau in [0.1, 0.3, 1.0, 3.0, 10.0]:
        h, m = draft_features(z, tau)
        h2, m2 = draft_features(z + 123.25, tau)           # shift
        h3, m3 = draft_features(z / tau, 1.0)              # temperature folds into z
        assert (h2, m2) == pytest.approx((h, m), rel=1e-9)
        assert (h3, m3) == pytest.approx((h, m), rel=1e-9)
        assert -math.log2(m) <= h + 1e-12                  # min-entropy <= Shannon entropy
        assert h <= math.log2(finite) + 1e-12              # support bound
        assert h > prev                                    # entropy rises with temperature
        prev = h


def test_faulty_rows_raise():
    for z in ([0.0, np.nan], [0.0, np.inf], [NEG, NEG]):
        with pytest.raises(ValueError):
            draft_features(np.array(z), 1.0)


def test_verify_reports_features_of_kept_draft_rows():
    rng = np.random.default_rng(2)
    n, k, V = 3, 3, 50
    kept = np.array([2, 0, 3])
    cu = np.concatenate([[0], np.cumsum(kept + 1)])
    target = rng.normal(0, 2, (int(cu[-1]), V))
    draft = rng.normal(0, 2, (n * k, V))
    toks = rng.integers(0, V, (n, k))
    res = oracle.verify(target, draft, toks, cu, k, V, oracle.STOCHASTIC, 0.8)
    for r in range(n):
        for j in range(k):
            if j < kept[r]:
                want = draft_features(draft[r * k + j], 0.8)
                assert (res["q_entropy"][r, j], res["q_max"][r, j]) == pytest.approx(want)
            else:
                assert res["q_entropy"][r, j] == -1 and res["q_max"][r, j] == -1
    g = oracle.verify(target, None, toks, cu, k, V, oracle.GREEDY, 1.0)
    assert (g["q_entropy"] == -1).all() and (g["q_max"] == -1).all()
