"""Helpers for the GPU-vs-oracle parity tests (not a test module).

Inputs come from the seeded generators in ``workloads``; expected values come
from ``oracle`` only.  The HIP path is reached through the binding, i.e.
through the C ABI.

Comparison rules:
* bit-exact: budget, kept counts, survival bits, cu_rows, row maps, packed
  tokens, greedy tokens and accepted lengths, device error bits, the accepted
  draft prefix;
* p(d), q(d): relative 1e-5, plus two fp32 subnormal ulps (2**-148) for values
  below fp32's normal range, where relative 1e-5 cannot be represented;
  residual mass W = sum max(0, p - q): relative 1e-5 plus RESID_KAPPA *
  (P+ + Q+), P+ and Q+ the masses of p and q over the ids where p > q (or
  p - q lies within that allowance of 0, either sign).  W is
  a difference of fp32 probabilities, so each p_x and q_x brings its own
  fp32 error into it, however small W is: RESID_KAPPA = 2^-21 allows 4 ulps
  (at fp32's 2^-23 spacing) per probability: the exp2 instruction's 1 ulp,
  the rounding of the exponent of a term that carries mass (|t| < 8: at most
  1.4 ulps), the normalisations (1) and the fp32 row sums (typically below
  1).  Over 1420 residual draws on 325 random shapes the kernel needed at
  most 2^-22.7;
* a stochastic accept decision may differ only where |u - p/q| < 1e-5 (then
  the oracle is replayed with the GPU's accepted length and every overridden
  decision must lie in that band);
* a stochastic token may differ only where the oracle's v * W lies within
  the band that the probability tolerance leaves on the cumulative weights,
  at every boundary between the two ids (``cdf_band``), and the GPU's id must
  carry positive weight (up to that tolerance for a residual);
* a residual whose oracle mass lies within that fp32 allowance of 0 may be
  empty to the kernel, so the zero-mass fallback (a draw from p at that row)
  may apply: the GPU's id then only has to lie in p's support;
* draft-row features: the largest probability relative 1e-5 (the same
  exp2-over-sum shape as q(d), never subnormal: it is at least 1/V); the
  entropy in bits absolute 1e-4 plus relative 1e-5 (log2 S minus a ratio of
  fp32 sums whose per-thread offsets are merged with a few roundings each).
"""

import numpy as np
import torch

import adaptive_draft_verification_amd as sv
import oracle
import workloads

U_BAND = 1e-5
CDF_BAND = 1e-5
P_RTOL = 1e-5
RESID_KAPPA = 2.0 ** -21  # per probability, in units of the probability
P_ATOL = 2.0 ** -148  # two fp32 subnormal ulps
H_ATOL = 1e-4         # bits
H_RTOL = 1e-5


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def logits_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


# ------------------------------------------------------------------ budget

def gpu_budget(conf, draft_len, cost, t_base, n_bonus):
    """sv_budget_select with every output pre-filled with a sentinel (-7, NaN), so
    that a value the kernels fail to write cannot pass on stale memory."""
    conf = np.asarray(conf, np.float32)
    n, k = conf.shape
    out = dict(kept=torch.full((n,), -7, dtype=torch.int32, device="cuda"),
               budget=torch.full((1,), -7, dtype=torch.int32, device="cuda"),
               survival=torch.full((n, k), float("nan"), dtype=torch.float32, device="cuda"),
               dev_error=torch.zeros(1, dtype=torch.int32, device="cuda"))
    ws = torch.empty(max(1, sv.sv_budget_workspace_bytes(n, k)), dtype=torch.uint8,
                     device="cuda")
    sv.sv_budget_select(to_dev(conf), to_dev(np.asarray(draft_len, np.int32)),
                        to_dev(np.asarray(cost, np.float32)), t_base, n_bonus, out["kept"],
                        out["budget"], out["survival"], out["dev_error"], ws=ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_budget(conf, draft_len, k_max, cost, t_base, n_bonus):
    g = gpu_budget(conf, draft_len, cost, t_base, n_bonus)
    o = oracle.budget_select(conf, draft_len, k_max, cost, t_base, n_bonus)
    assert int(g["budget"][0]) == o["budget"], (int(g["budget"][0]), o["budget"])
    np.testing.assert_array_equal(g["kept"], o["kept"])
    np.testing.assert_array_equal(g["survival"].view(np.uint32), o["survival"].view(np.uint32))
    assert int(g["dev_error"][0]) == o["dev_error"]
    return o


def check_allocate(conf, draft_len, k_max, budget):
    """Allocation of a given budget: kept counts, the clamped B, survival bits."""
    conf = np.asarray(conf, np.float32).reshape(len(draft_len), k_max)
    n = len(draft_len)
    g = dict(kept=torch.full((n,), -7, dtype=torch.int32, device="cuda"),
             budget_used=torch.full((1,), -7, dtype=torch.int32, device="cuda"),
             survival=torch.full((n, k_max), float("nan"), dtype=torch.float32, device="cuda"),
             dev_error=torch.zeros(1, dtype=torch.int32, device="cuda"))
    ws = torch.empty(max(1, sv.sv_budget_workspace_bytes(n, k_max)), dtype=torch.uint8,
                     device="cuda")
    sv.sv_budget_allocate(to_dev(conf), to_dev(np.asarray(draft_len, np.int32)),
                          to_dev(np.array([budget], np.int32)), g["kept"], g["budget_used"],
                          g["survival"], g["dev_error"], ws=ws)
    torch.cuda.synchronize()
    o = oracle.budget_allocate(conf, draft_len, k_max, budget)
    np.testing.assert_array_equal(g["kept"].cpu().numpy(), o["kept"])
    assert int(g["budget_used"].cpu()[0]) == o["budget_used"]
    np.testing.assert_array_equal(g["survival"].cpu().numpy().view(np.uint32),
                                  o["survival"].view(np.uint32))
    assert int(g["dev_error"].cpu()[0]) == o["dev_error"]
    return o


def check_uniform_k(conf, draft_len, k_max, cost, t_base, n_bonus):
    """Uniform draft length: K*, kept counts and every K's fp64 score exact."""
    conf = np.asarray(conf, np.float32).reshape(len(draft_len), k_max)
    g = sv.uniform_k_select(to_dev(conf), to_dev(np.asarray(draft_len, np.int32)),
                            to_dev(np.asarray(cost, np.float32)), t_base, n_bonus)
    torch.cuda.synchronize()
    o = oracle.uniform_k_select(conf, draft_len, k_max, cost, t_base, n_bonus)
    assert int(g["k"].cpu()[0]) == o["k"], (int(g["k"].cpu()[0]), o["k"])
    np.testing.assert_array_equal(g["kept"].cpu().numpy(), o["kept"])
    np.testing.assert_array_equal(g["scores"].cpu().numpy(), np.array(o["scores"], np.float64))
    assert int(g["dev_error"].cpu()[0]) == o["dev_error"]
    return o


# -------------------------------------------------------------------- pack

def check_pack(kept, last_token, draft_tokens, k_max):
    draft_tokens = np.asarray(draft_tokens, np.int32).reshape(len(kept), k_max)
    g = sv.pack_varlen(to_dev(np.asarray(kept, np.int32)), to_dev(np.asarray(last_token, np.int32)),
                       to_dev(draft_tokens))
    torch.cuda.synchronize()
    o = oracle.pack_varlen(kept, last_token, draft_tokens, k_max)
    for key in ("cu_rows", "row_req", "row_pos", "packed_tokens"):
        np.testing.assert_array_equal(g[key].cpu().numpy(), o[key], err_msg=key)
    assert int(g["dev_error"].cpu()[0]) == o["dev_error"]
    return o


# ------------------------------------------------------------------ verify

def gpu_verify(target, draft, draft_tokens, cu_rows, k_max, mode, tau, dtype, seed=0, step=0,
               vocab=None, target_ld=None, draft_ld=None, features=False):
    """Run sv_verify on host arrays (fp32 holding the exact logit values).

    target_ld / draft_ld > vocab place rows at a wider stride (the extra
    columns hold NaN that must never be read).  features: also ask for the
    draft-row features."""
    V = target.shape[1] if vocab is None else vocab

    def widen(a, ld):
        if ld is None or ld == a.shape[1]:
            return a
        out = np.full((a.shape[0], ld), np.nan, dtype=np.float32)
        out[:, : a.shape[1]] = a
        return out

    t = to_dev(widen(target, target_ld), dtype)
    d = None if draft is None else to_dev(widen(draft, draft_ld), dtype)
    out = sv.verify(t, d, to_dev(np.asarray(draft_tokens, np.int32)),
                    to_dev(np.asarray(cu_rows, np.int32)),
                    sv.SV_GREEDY if mode == "greedy" else sv.SV_STOCHASTIC, tau, seed, step,
                    vocab=V, features=features)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_verify(g, target, draft, draft_tokens, cu_rows, k_max, vocab, mode, tau, seed=0,
                   step=0):
    """Check GPU outputs against the oracle; returns counts of band cases."""
    om = oracle.GREEDY if mode == "greedy" else oracle.STOCHASTIC
    o = oracle.verify(target, draft, draft_tokens, cu_rows, k_max, vocab, om, tau, seed, step)
    stats = dict(requests=len(cu_rows) - 1, u_band=0, cdf_band=0, degenerate=0)
    assert int(g["dev_error"][0]) == o["dev_error"], (int(g["dev_error"][0]), o["dev_error"])
    n = len(cu_rows) - 1
    draft_tokens = np.asarray(draft_tokens).reshape(n, k_max)
    feats = "q_entropy" in g
    if mode == "greedy":
        np.testing.assert_array_equal(g["tokens"], o["tokens"])
        np.testing.assert_array_equal(g["accepted"], o["accepted"])
        assert (g["p_draft"] == -1).all() and (g["q_draft"] == -1).all()
        assert (g["residual_mass"] == -1).all()
        if feats:
            assert (g["q_entropy"] == -1).all() and (g["q_max"] == -1).all()
        return stats
    for r in range(n):
        res = o["per_request"][r]
        if res is None or res["fault"]:
            assert g["accepted"][r] == -1 and (g["tokens"][r] == -1).all()
            assert (g["p_draft"][r] == -1).all() and (g["q_draft"][r] == -1).all()
            assert g["residual_mass"][r] == -1
            if feats:
                assert (g["q_entropy"][r] == -1).all() and (g["q_max"][r] == -1).all()
            continue
        b = int(cu_rows[r + 1] - cu_rows[r] - 1)
        # probabilities of the draft ids
        np.testing.assert_allclose(g["p_draft"][r, :b], res["p_d"], rtol=P_RTOL, atol=P_ATOL,
                                   err_msg=f"p(d) request {r}")
        np.testing.assert_allclose(g["q_draft"][r, :b], res["q_d"], rtol=P_RTOL, atol=P_ATOL,
                                   err_msg=f"q(d) request {r}")
        assert (g["p_draft"][r, b:] == -1).all() and (g["q_draft"][r, b:] == -1).all()
        if feats:
            np.testing.assert_allclose(g["q_entropy"][r, :b], res["q_entropy"], rtol=H_RTOL,
                                       atol=H_ATOL, err_msg=f"entropy request {r}")
            np.testing.assert_allclose(g["q_max"][r, :b], res["q_max"], rtol=P_RTOL, atol=0,
                                       err_msg=f"largest probability request {r}")
            assert (g["q_entropy"][r, b:] == -1).all() and (g["q_max"][r, b:] == -1).all()
        Lg = int(g["accepted"][r])
        assert 0 <= Lg <= b
        replayed = Lg != res["L"]
        if replayed:
            # first differing decision must sit in the u band; replay with the GPU's L
            rep = oracle.verify_request(r, _rows_t(target, cu_rows, r, b),
                                        _rows_d(draft, r, k_max, b), draft_tokens[r], b, vocab,
                                        om, tau, seed, step, forced_l=Lg)
            assert rep["overridden"], r
            for _j, gap in rep["overridden"]:
                assert gap < U_BAND, (r, _j, gap)
            stats["u_band"] += 1
            res = rep
        # accepted prefix is the draft ids themselves
        np.testing.assert_array_equal(g["tokens"][r, :Lg], draft_tokens[r, :Lg])
        assert (g["tokens"][r, Lg + 1:] == -1).all()
        gt, ot = int(g["tokens"][r, Lg]), int(res["tokens"][Lg])
        resid_floor = 0.0
        if Lg < b:
            want = res["residual_mass"]
            p_l = oracle.row_probs(target[int(cu_rows[r]) + Lg, :vocab], tau)
            q_l = oracle.row_probs(draft[r * k_max + Lg, :vocab], tau)
            resid_floor = resid_allowance(p_l, q_l)
            assert abs(g["residual_mass"][r] - want) <= P_RTOL * want + resid_floor, \
                (r, g["residual_mass"][r], want, resid_floor)
        else:
            assert g["residual_mass"][r] == -1
        if gt != ot:
            if Lg < b and res["residual_mass"] <= resid_floor:
                # a residual within the fp32 allowance of empty: the kernel may
                # find no mass and take the zero-mass fallback (a draw from p)
                p_l = oracle.row_probs(target[int(cu_rows[r]) + Lg, :vocab], tau)
                assert 0 <= gt < vocab and p_l[gt] > 0, (r, gt)
                stats["degenerate"] += 1
                continue
            full = oracle.verify_request(r, _rows_t(target, cu_rows, r, b),
                                         _rows_d(draft, r, k_max, b), draft_tokens[r], b, vocab,
                                         om, tau, seed, step, forced_l=Lg, keep_weights=True)
            w, v = full["weights"], full["v"]
            assert 0 <= gt < vocab, (r, gt)
            p_l = oracle.row_probs(target[int(cu_rows[r]) + Lg, :vocab], tau)
            if Lg < b:  # residual max(0, p - q) of target row Lg and draft row Lg
                q_l = oracle.row_probs(draft[r * k_max + Lg, :vocab], tau)
                assert p_l[gt] > 0 and p_l[gt] >= q_l[gt] * (1 - 2 * P_RTOL), (r, gt)
            else:       # bonus draw from p
                q_l = np.zeros_like(p_l)
                assert p_l[gt] > 0, (r, gt)
            lo, hi = min(gt, ot), max(gt, ot)
            band = cdf_band(p_l, q_l, v)
            c = np.cumsum(w)
            assert np.all(np.abs(c[lo:hi] - v * c[-1]) <= band[lo:hi]), (r, gt, ot)
            stats["cdf_band"] += 1
    return stats


def resid_allowance(p, q):
    """Absolute part of the residual-mass tolerance: RESID_KAPPA * (P+ + Q+),
    the fp32 errors of the probabilities that the sum max(0, p - q) adds up,
    over every id whose term the kernel may count: p > q, or p - q within
    those errors of 0 (where rounding can give the difference either sign)."""
    pos = p - q > -RESID_KAPPA * (p + q)
    return RESID_KAPPA * float(p[pos].sum() + q[pos].sum())


def cdf_band(p, q, v):
    """Per-boundary tolerance of a draw's cumulative weights, in units of p's mass.

    The draw's weights are max(0, p - q) (a residual) or p (a bonus draw, q = 0).
    With every probability allowed a relative error CDF_BAND (the tolerance of
    p(d) and q(d)), a weight may move by CDF_BAND * (p_x + q_x), the running sum
    C(x) by CDF_BAND * (P(x) + Q(x)) with P, Q the running sums of p and q, and
    the target v * W by v * CDF_BAND * (P + Q over the whole row).  A boundary x
    is ambiguous when |C(x) - v * W| is within the sum of the two.
    """
    P, Q = np.cumsum(p), np.cumsum(q)
    return CDF_BAND * (P + Q + v * (P[-1] + Q[-1]))


def _rows_t(target, cu_rows, r, b):
    lo = int(cu_rows[r])
    return [target[lo + j] for j in range(b + 1)]


def _rows_d(draft, r, k_max, b):
    if draft is None:
        return []
    return [draft[r * k_max + j] for j in range(b)]


def workload_inputs(w, kept, mode):
    """Packed target, padded draft, draft ids and cu_rows (oracle pack) for `kept`."""
    toks = w.draft_tokens(mode)
    pk = oracle.pack_varlen(kept, w.last_token, toks, w.k_max)
    target = workloads.assemble_target(w, pk["cu_rows"], kept)
    draft = workloads.assemble_draft(w, kept) if mode != "greedy" else None
    return target, draft, toks, pk["cu_rows"]
