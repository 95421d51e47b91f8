"""Pins for the oracle's pack and verify (CPU only).

What fixes the answers here is not the oracle itself:
* hand-derived golden fixtures under tests/golden/ (each with its derivation);
* exact enumeration on a 32-token vocabulary over the full 2**-24 uniform
  grid: the law of the emitted token must equal the target distribution
  (FOS page "추측 디코딩과 vLLM 적응형 검증", section "속도, 메모리, 정확도에
  주는 영향", row 정확도: rejection sampling keeps the target's distribution);
* chi-square over 10**6 seeded end-to-end trials, per position, and the
  closed forms alpha = sum min(p, q), P(L >= j) = prod_{i<j} alpha_i;
* the identity residual mass = 1 - sum min(p, q) = 0.5 * |p - q|_1;
* planted mistakes (in the oracle, on the CPU) that the enumeration must catch.
"""

import json
import math
import os
import sys

import numpy as np
import pytest
import scipy.special
from scipy import stats

import oracle
import workloads

overify = sys.modules["oracle.verify"]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GRID = 2 ** 24


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def logits_of(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


# --------------------------------------------------------------------------- pack

def test_pack_golden():
    g = load("pack_small.json")
    res = oracle.pack_varlen(g["kept"], g["last_token"], g["draft_tokens"], g["k_max"])
    for key in ("cu_rows", "row_req", "row_pos", "packed_tokens"):
        np.testing.assert_array_equal(res[key], g[key])
    assert res["dev_error"] == 0
    assert len(res["row_req"]) == (g["k_max"] + 1) * len(g["kept"])


def test_pack_bad_kept_is_flagged_and_clamped():
    res = oracle.pack_varlen([5, -1], [1, 2], [[3, 4], [5, 6]], 2)
    assert res["dev_error"] == oracle.DEV_BAD_KEPT
    np.testing.assert_array_equal(res["cu_rows"], [0, 3, 4])
    np.testing.assert_array_equal(res["packed_tokens"], [1, 3, 4, 2, -1, -1])


def test_pack_full_k_is_uniform():
    n, k = 7, 3
    res = oracle.pack_varlen([k] * n, list(range(n)), np.arange(n * k).reshape(n, k), k)
    np.testing.assert_array_equal(res["cu_rows"], np.arange(n + 1) * (k + 1))
    assert (res["row_req"] >= 0).all()


# ------------------------------------------------------------------------ greedy

def test_greedy_golden():
    g = load("verify_greedy_small.json")
    target = np.array([[float(x) for x in row] for row in g["target"]])
    res = oracle.verify(target, None, g["draft_tokens"], g["cu_rows"], g["k_max"], g["vocab"],
                        oracle.GREEDY, 1.0)
    np.testing.assert_array_equal(res["tokens"], g["tokens"])
    np.testing.assert_array_equal(res["accepted"], g["accepted"])
    assert res["dev_error"] == 0
    assert (res["p_draft"] == -1).all() and (res["residual_mass"] == -1).all()


def test_greedy_invariants_random():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n, k, V = 5, 4, 16
        kept = rng.integers(0, k + 1, n)
        cu = np.concatenate([[0], np.cumsum(kept + 1)])
        target = np.round(rng.normal(0, 1, (cu[-1], V)) * 2) / 2  # many ties
        argm = [int(np.flatnonzero(row == row.max())[0]) for row in target]
        drafts = np.where(rng.uniform(size=(n, k)) < 0.6,
                          np.array([[argm[min(cu[r] + j, cu[r + 1] - 1)] for j in range(k)]
                                    for r in range(n)]),
                          rng.integers(0, V, (n, k)))
        res = oracle.verify(target, None, drafts, cu, k, V, oracle.GREEDY, 1.0)
        for r in range(n):
            L = res["accepted"][r]
            assert 0 <= L <= kept[r]
            assert list(res["tokens"][r, :L]) == list(drafts[r, :L])
            assert res["tokens"][r, L] == argm[cu[r] + L]
            assert all(drafts[r, j] == argm[cu[r] + j] for j in range(L))
            if L < kept[r]:
                assert drafts[r, L] != argm[cu[r] + L]
            assert (res["tokens"][r, L + 1:] == -1).all()


# -------------------------------------------------------------- stochastic rule

def test_stochastic_golden(monkeypatch):
    g = load("verify_stochastic_cases.json")
    for case in g["cases"]:
        us, vs = case["u"], case["v"]
        monkeypatch.setattr(overify, "uniforms",
                            lambda seed, r, j, step, us=us, vs=vs: (us[j], vs[j]))
        b = len(case["draft"])
        res = oracle.verify_request(0, [logits_of(p) for p in case["p"]],
                                    [logits_of(q) for q in case["q"]], case["draft"], b, 4,
                                    oracle.STOCHASTIC, 1.0, 0, 0)
        assert res["tokens"] == case["tokens"], case["name"]
        assert res["L"] == case["accepted"], case["name"]
        assert res["residual_mass"] == pytest.approx(case["residual_mass"], abs=1e-12)


def test_residual_mass_identity_and_zero_mass_fallback():
    rng = np.random.default_rng(11)
    for _ in range(100):
        p = rng.dirichlet(np.ones(32) * 0.3)
        q = rng.dirichlet(np.ones(32) * 0.3)
        w, mass = oracle.residual_weights(p, q)
        assert mass == pytest.approx(1 - np.minimum(p, q).sum(), abs=1e-12)
        assert mass == pytest.approx(0.5 * np.abs(p - q).sum(), abs=1e-12)
        assert (w >= 0).all()
    w, mass = oracle.residual_weights(p, p.copy())
    assert mass == 0.0 and np.array_equal(w, p)


def test_inverse_cdf_edges():
    w = np.array([0.0, 0.25, 0.0, 0.75, 0.0])
    assert oracle.inverse_cdf(w, 0.0) == 1
    assert oracle.inverse_cdf(w, 0.25) == 3        # strict '>' skips the boundary
    assert oracle.inverse_cdf(w, 1.0 - 2 ** -24) == 3
    assert oracle.inverse_cdf(w, 1.0) == 3         # no id exceeds: last positive id
    assert oracle.inverse_cdf(np.array([1.0]), 0.5) == 0


def accept_fraction(p_d, q_d):
    """Share of the 2**24 u-grid that the oracle's accept() accepts (bisection:
    accept is monotone in u)."""
    lo, hi = 0, GRID  # accept(lo / GRID) is known true iff any is
    if not oracle.accept(0.0, p_d, q_d):
        return 0.0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if oracle.accept(mid / GRID, p_d, q_d):
            lo = mid
        else:
            hi = mid
    return hi / GRID


def draw_law(w):
    """Law of oracle.inverse_cdf(w, v) for v uniform on the 2**-24 grid."""
    V = len(w)
    first = np.zeros(V + 1, dtype=np.int64)  # first grid index whose draw is >= x
    for x in range(V + 1):
        lo, hi = -1, GRID  # draw(hi) >= x, draw(lo) < x
        if x == 0:
            first[x] = 0
            continue
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if oracle.inverse_cdf(w, mid / GRID) >= x:
                hi = mid
            else:
                lo = mid
        first[x] = hi
    first[V] = GRID
    return np.diff(first) / GRID


def emitted_law(p, q):
    """Law of the token emitted at one position when the draft is drawn from q."""
    V = len(p)
    w, _ = oracle.residual_weights(p, q)
    res_law = draw_law(w)
    law = np.zeros(V)
    for d in range(V):
        if q[d] == 0:
            continue
        a = accept_fraction(p[d], q[d])
        law[d] += q[d] * a
        law += q[d] * (1 - a) * res_law
    return law


@pytest.mark.parametrize("seed", range(6))
def test_exact_enumeration_preserves_target_law(seed):
    rng = np.random.default_rng(seed)
    V = 32
    conc = [1.0, 0.2, 5.0, 0.5, 1.0, 0.05][seed]
    p = rng.dirichlet(np.ones(V) * conc)
    q = rng.dirichlet(np.ones(V) * conc)
    if seed == 4:
        q[:8] = 0  # drafts never propose ids 0..7
        q /= q.sum()
    law = emitted_law(p, q)
    np.testing.assert_allclose(law, p, atol=4e-6)
    # the bonus draw from p itself
    np.testing.assert_allclose(draw_law(p), p, atol=4e-6)
    # acceptance probability alpha = sum min(p, q)
    alpha = sum(q[d] * accept_fraction(p[d], q[d]) for d in range(V) if q[d] > 0)
    assert alpha == pytest.approx(np.minimum(p, q).sum(), abs=4e-6)


@pytest.mark.parametrize("mutation", ["residual_sign", "inverted_ratio", "no_clip",
                                      "bonus_from_q"])
def test_enumeration_catches_planted_mistakes(monkeypatch, mutation):
    """Plausible slips planted in the oracle (CPU only) must break the law."""
    rng = np.random.default_rng(99)
    V = 32
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    if mutation == "residual_sign":
        monkeypatch.setattr(oracle, "residual_weights",
                            lambda p_, q_: (np.maximum(0, q_ - p_), 0.0))
    elif mutation == "inverted_ratio":
        monkeypatch.setattr(oracle, "accept", lambda u, pd, qd: u < qd / pd)
    elif mutation == "no_clip":
        monkeypatch.setattr(oracle, "residual_weights",
                            lambda p_, q_: (np.abs(p_ - q_), 0.0))
    if mutation == "bonus_from_q":
        bad = draw_law(q)
        assert np.abs(bad - p).max() > 1e-3
        return
    law = emitted_law(p, q)
    assert np.abs(law - p).max() > 1e-3


# -------------------------------------------------------- chi-square, 10**6 trials

V_CHI, B_CHI, N_CHI = 32, 3, 10 ** 6


def _chi_setup():
    rng = np.random.default_rng(2024)
    ps = [rng.dirichlet(np.ones(V_CHI) * 0.7) for _ in range(B_CHI + 1)]
    qs = [0.5 * ps[j] + 0.5 * rng.dirichlet(np.ones(V_CHI) * 0.7) for j in range(B_CHI)]
    return ps, qs


def _chi_worker(args):
    r0, r1, drafts = args
    ps, qs = _chi_setup()
    tr = [logits_of(p) for p in ps]
    dr = [logits_of(q) for q in qs]
    toks = np.full((r1 - r0, B_CHI + 1), -1, dtype=np.int32)
    lens = np.zeros(r1 - r0, dtype=np.int32)
    for i, r in enumerate(range(r0, r1)):
        res = oracle.verify_request(r, tr, dr, drafts[i], B_CHI, V_CHI, oracle.STOCHASTIC,
                                    1.0, 4242, 17)
        lens[i] = res["L"]
        toks[i, : len(res["tokens"])] = res["tokens"]
    return toks, lens


def test_chi_square_million_trials():
    import multiprocessing as mp
    ps, qs = _chi_setup()
    drafter = np.random.default_rng(77)
    drafts = np.stack([np.searchsorted(np.cumsum(q), drafter.random(N_CHI), side="right")
                       for q in qs], axis=1).clip(0, V_CHI - 1)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    chunks = np.linspace(0, N_CHI, workers * 4 + 1).astype(int)
    jobs = [(int(a), int(b), drafts[a:b]) for a, b in zip(chunks[:-1], chunks[1:])]
    with mp.get_context("fork").Pool(workers) as pool:
        parts = pool.map(_chi_worker, jobs)
    toks = np.concatenate([t for t, _ in parts])
    lens = np.concatenate([l for _, l in parts])
    alphas = [np.minimum(p, q).sum() for p, q in zip(ps, qs)]
    for j in range(B_CHI + 1):
        reached = lens >= j
        expect_reach = np.prod(alphas[:j]) if j else 1.0
        nr = reached.sum()
        sd = np.sqrt(N_CHI * expect_reach * (1 - expect_reach)) + 1e-9
        assert abs(nr - N_CHI * expect_reach) < 5 * sd + 1
        counts = np.bincount(toks[reached, j], minlength=V_CHI)
        exp = ps[j] * nr
        keep = exp >= 5
        f_obs = np.append(counts[keep], counts[~keep].sum())
        f_exp = np.append(exp[keep], exp[~keep].sum())
        if f_exp[-1] == 0:
            f_obs, f_exp = f_obs[:-1], f_exp[:-1]
        pval = stats.chisquare(f_obs, f_exp * f_obs.sum() / f_exp.sum()).pvalue
        assert pval > 1e-4, (j, pval)
    mean_l = lens.mean()
    expect_l = sum(np.prod(alphas[:j]) for j in range(1, B_CHI + 1))
    assert abs(mean_l - expect_l) < 5 * lens.std() / np.sqrt(N_CHI)


# --------------------------------------------------------------- faults, layout

def test_faults_mark_the_request():
    rng = np.random.default_rng(1)
    V, k = 16, 2
    cu = [0, 3, 6, 9, 12]
    target = rng.normal(0, 1, (12, V))
    draft = rng.normal(0, 1, (8, V))
    toks = np.array([[1, 2], [3, 99], [0, 0], [5, 6]])
    target[6 + 1, 4] = np.nan        # request 2, row 1
    draft[3 * k + 1, :] = -np.inf    # request 3, draft row 1: no mass
    res = oracle.verify(target, draft, toks, cu, k, V, oracle.STOCHASTIC, 1.0, 0, 0)
    assert res["dev_error"] == oracle.DEV_BAD_TOKEN | oracle.DEV_NONFINITE
    assert res["accepted"][0] >= 0
    for r in (1, 2, 3):
        assert res["accepted"][r] == -1 and (res["tokens"][r] == -1).all()
        assert (res["p_draft"][r] == -1).all()
    # greedy reads no draft rows; request 3 is fine there, request 1 still bad
    res = oracle.verify(target, None, toks, cu, k, V, oracle.GREEDY, 1.0)
    assert res["dev_error"] == oracle.DEV_BAD_TOKEN | oracle.DEV_NONFINITE
    assert res["accepted"][3] >= 0
    # inconsistent offsets
    res = oracle.verify(target, draft, toks, [0, 3, 2, 9, 13], k, V, oracle.STOCHASTIC, 1.0)
    assert res["dev_error"] & oracle.DEV_BAD_CU_ROWS
    assert res["accepted"][1] == -1 and res["accepted"][3] == -1


def test_masked_logits_are_legal():
    z = np.array([0.0, -np.inf, 1.0, -np.inf])
    assert not oracle.row_is_faulty(z)
    p = oracle.row_probs(z, 0.5)
    assert p[1] == 0 and p[3] == 0 and p.sum() == pytest.approx(1.0)
    assert oracle.row_is_faulty(np.array([-np.inf, -np.inf]))
    assert oracle.row_is_faulty(np.array([0.0, np.inf]))


def test_forced_replay_reports_overrides():
    w = workloads.make("tiny")
    kept = w.draft_len
    pk = oracle.pack_varlen(kept, w.last_token, w.draft_tokens("stochastic"), w.k_max)
    target = workloads.assemble_target(w, pk["cu_rows"], kept)
    draft = workloads.assemble_draft(w, kept)
    base = oracle.verify(target, draft, w.draft_tokens("stochastic"), pk["cu_rows"], w.k_max,
                         w.vocab, oracle.STOCHASTIC, w.tau)
    assert base["dev_error"] == 0
    r = 0
    L = int(base["accepted"][r])
    forced_l = (L + 1) % (w.k_max + 1)
    rep = oracle.verify(target, draft, w.draft_tokens("stochastic"), pk["cu_rows"], w.k_max,
                        w.vocab, oracle.STOCHASTIC, w.tau, forced={r: forced_l})
    assert rep["accepted"][r] == forced_l
    assert len(rep["per_request"][r]["overridden"]) >= 1


# ------------------------------------------------------------------ temperature
#
# The pages never mention a temperature; the verify step scales target and
# draft logits alike, p = softmax(z / tau), q = softmax(z_draft / tau).  What
# pins that scaling independently of the oracle's own code: two-point rows
# whose softmax has a closed form, scipy's softmax on random rows, rows built
# as tau * log(w) (whose law at tau is w / sum w by construction), and the
# exact law of the emitted token at tau != 1 — which equals the target law only
# if p and q are both taken at tau.

def test_row_probs_two_point_closed_form():
    # z = (0, ln 3): z / tau = (0, ln 3 / tau), so p = (1, 3^(1/tau)) / (1 + 3^(1/tau))
    ln3 = math.log(3.0)
    np.testing.assert_allclose(oracle.row_probs([0.0, ln3], 0.5), [0.1, 0.9], rtol=1e-13)
    r3 = math.sqrt(3.0)
    np.testing.assert_allclose(oracle.row_probs([0.0, ln3], 2.0),
                               [1 / (1 + r3), r3 / (1 + r3)], rtol=1e-13)
    # a masked id keeps probability 0 at any temperature
    np.testing.assert_allclose(oracle.row_probs([0.0, -np.inf, ln3], 0.25),
                               [1 / 82, 0.0, 81 / 82], rtol=1e-13)
    # tau -> 0 concentrates on the argmax, large tau flattens
    p = oracle.row_probs([0.0, 1.0, 2.0], 0.01)
    assert p[2] == 1.0
    assert p[1] == pytest.approx(math.exp(-100.0), rel=1e-12)
    assert p[0] == pytest.approx(math.exp(-200.0), rel=1e-12)
    np.testing.assert_allclose(oracle.row_probs([0.0, 1.0, 2.0], 1e6), [1 / 3] * 3, rtol=1e-5)


@pytest.mark.parametrize("tau", [0.05, 0.3, 0.7, 1.8])
def test_row_probs_matches_scipy_softmax(tau):
    rng = np.random.default_rng(int(tau * 100))
    z = rng.normal(0, 3, 5000)
    z[rng.uniform(size=z.size) < 0.05] = -np.inf
    want = scipy.special.softmax(z / tau)
    np.testing.assert_allclose(oracle.row_probs(z, tau), want, rtol=1e-10, atol=1e-300)


@pytest.mark.parametrize("tau", [0.25, 0.7, 3.0])
def test_row_probs_of_scaled_log_weights(tau):
    rng = np.random.default_rng(5)
    w = rng.dirichlet(np.ones(64) * 0.5)
    w[:5] = 0.0
    w /= w.sum()
    np.testing.assert_allclose(oracle.row_probs(tau * logits_of(w), tau), w, rtol=1e-9,
                               atol=1e-300)


V_TAU = 16


def _tau_case(seed):
    rng = np.random.default_rng(seed)
    p0 = rng.dirichlet(np.ones(V_TAU) * 0.6)
    q0 = rng.dirichlet(np.ones(V_TAU) * 0.6)
    q0[:3] = 0.0  # the drafter never proposes ids 0..2
    q0 /= q0.sum()
    p0[5] = 0.0   # the target never emits id 5
    p0 /= p0.sum()
    return p0, q0


def _draws_through_verify(monkeypatch, trows, drows, dtoks, b, tau):
    """Token and accepted length of oracle.verify_request as functions of (u, v)."""
    def run(u, v):
        monkeypatch.setattr(overify, "uniforms", lambda seed, r, j, step: (u, v))
        res = oracle.verify_request(0, trows, drows, dtoks, b, V_TAU, oracle.STOCHASTIC, tau,
                                    0, 0)
        return res["L"], res["tokens"][-1]
    return run


def _grid_law(token_of_v):
    """Law over ids of a token that is a non-decreasing function of v on the 2**-24 grid."""
    first = np.zeros(V_TAU + 1, dtype=np.int64)
    for x in range(1, V_TAU + 1):
        lo, hi = -1, GRID
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if token_of_v(mid / GRID) >= x:
                hi = mid
            else:
                lo = mid
        first[x] = hi
    first[V_TAU] = GRID
    return np.diff(first) / GRID


def _emitted_law_at_tau(monkeypatch, p0, q0, tau):
    """Law of the emitted token of a one-draft request whose logits are tau * log p0 and
    tau * log q0, the draft drawn from q0, every decision taken by the oracle at tau."""
    t0 = tau * logits_of(p0)
    d0 = tau * logits_of(q0)
    t1 = t0.copy()  # bonus row (its law is checked on its own below)
    law = np.zeros(V_TAU)
    res_law = None
    for d in range(V_TAU):
        if q0[d] == 0:
            continue
        run = _draws_through_verify(monkeypatch, [t0, t1], [d0], [d], 1, tau)
        # acceptance share of the u grid (accepted iff L == 1; monotone in u)
        if run(0.0, 0.5)[0] != 1:
            a = 0.0
        else:
            lo, hi = 0, GRID
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if run(mid / GRID, 0.5)[0] == 1:
                    lo = mid
                else:
                    hi = mid
            a = hi / GRID
        law[d] += q0[d] * a
        if a < 1.0:
            if res_law is None:  # the residual law does not depend on d
                u_rej = (GRID - 1) / GRID
                assert run(u_rej, 0.5)[0] == 0
                res_law = _grid_law(lambda v: run(u_rej, v)[1])
            law += q0[d] * (1.0 - a) * res_law
    return law


def _bonus_law_at_tau(monkeypatch, p0, tau):
    run = _draws_through_verify(monkeypatch, [tau * logits_of(p0)], [], [], 0, tau)
    return _grid_law(lambda v: run(0.0, v)[1])


@pytest.mark.parametrize("tau", [0.5, 0.7, 1.8])
def test_exact_enumeration_at_temperature(monkeypatch, tau):
    """At tau != 1 the emitted token's law must be p = softmax(z / tau), for the
    first position and for the bonus draw (FOS "속도, 메모리, 정확도에 주는 영향",
    row 정확도: the output keeps the target's distribution)."""
    p0, q0 = _tau_case(int(tau * 10))
    np.testing.assert_allclose(_emitted_law_at_tau(monkeypatch, p0, q0, tau), p0, atol=4e-6)
    np.testing.assert_allclose(_bonus_law_at_tau(monkeypatch, p0, tau), p0, atol=4e-6)


@pytest.mark.parametrize("mutation", ["times_tau", "tau_ignored", "draft_at_one",
                                      "target_at_one"])
def test_temperature_enumeration_catches_planted_mistakes(monkeypatch, mutation):
    """Temperature slips planted in the oracle (CPU only) must break the law at tau = 0.5."""
    tau = 0.5
    p0, q0 = _tau_case(3)
    orig = overify.row_probs
    drafts = []

    def planted(z, t):
        is_draft = any(z is dr for dr in drafts)
        if mutation == "times_tau":
            return orig(np.asarray(z, dtype=np.float64) * t * t, t)  # z * tau
        if mutation == "tau_ignored":
            return orig(z, 1.0)
        if mutation == "draft_at_one" and is_draft:
            return orig(z, 1.0)
        if mutation == "target_at_one" and not is_draft:
            return orig(z, 1.0)
        return orig(z, t)

    real_request = overify.verify_request

    def spy(r, trows, drows, *args, **kw):
        drafts[:] = list(drows)
        return real_request(r, trows, drows, *args, **kw)

    monkeypatch.setattr(overify, "row_probs", planted)
    monkeypatch.setattr(oracle, "verify_request", spy)
    law = _emitted_law_at_tau(monkeypatch, p0, q0, tau)
    bonus = _bonus_law_at_tau(monkeypatch, p0, tau)
    worst = max(np.abs(law - p0).max(), np.abs(bonus - p0).max())
    assert worst > 1e-3, (mutation, worst)


def test_stochastic_golden_at_temperature(monkeypatch):
    """Hand-derived cases at tau != 1 (tests/golden/verify_stochastic_tau.json):
    logits tau * ln(w), so the law at tau is w."""
    g = load("verify_stochastic_tau.json")
    for case in g["cases"]:
        tau = case["tau"]
        us, vs = case["u"], case["v"]
        monkeypatch.setattr(overify, "uniforms",
                            lambda seed, r, j, step, us=us, vs=vs: (us[j], vs[j]))
        b = len(case["draft"])
        V = len(case["p"][0])
        res = oracle.verify_request(0, [tau * logits_of(p) for p in case["p"]],
                                    [tau * logits_of(q) for q in case["q"]], case["draft"], b,
                                    V, oracle.STOCHASTIC, tau, 0, 0)
        assert res["tokens"] == case["tokens"], case["name"]
        assert res["L"] == case["accepted"], case["name"]
        np.testing.assert_allclose(res["p_d"], case["p_d"], rtol=1e-12, err_msg=case["name"])
        np.testing.assert_allclose(res["q_d"], case["q_d"], rtol=1e-12, err_msg=case["name"])
        assert res["residual_mass"] == pytest.approx(case["residual_mass"], abs=1e-12)
