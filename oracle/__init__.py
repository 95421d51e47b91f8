"""Oracle for the batched speculative-decoding verify step — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU statement of what the
HIP library computes.  It exists to check the library, never to stand in for
it: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  It shares no code, header, table or constant
generator with ``adaptive_draft_verification_amd`` and imports nothing from it.

Pages the oracle follows (cited by title and section in every function):

* "추측 디코딩과 vLLM 적응형 검증" (Speculative decoding and vLLM adaptive
  verification), FOS Study blog, 2026-11-14.
* "vLLM DSpark을 활용한 적응형 검증(Adaptive Verification)" (agentlens).
* "Hardware-Aware Dynamic Speculative Decoding (DSD), feat. Cohere"
  (PyTorch Korea discussion forum).

Precision: floating-point work is fp64 (numpy) except where the library's
contract fixes another type on purpose — survival products are fp32 (the
ranking keys are fp32 bit patterns) and budget sums are exact integers in
units of 2**-40 (so the sum does not depend on summation order).

Parity pin status (what the oracle is checked against, in tests/):

* philox4x32_10 — pinned against rocRAND's Philox4x32-10 host code (a second,
  independent implementation) and by uniformity statistics.
* survival / expected tokens — pinned against the acceptance tables printed on
  the FOS page (per-position table, truncated-k table, 0.55**7 chain example).
* budget_select — pinned by exhaustive exact-rational search over every
  per-request allocation on small cases, by the truncated-k table read as a
  cost model, and by prefix-closure invariants.
* budget_allocate (a budget sized elsewhere, slots from the current
  confidences) — pinned by exhaustive exact-rational search (the kept slots
  carry the largest survival total of any prefix allocation of B slots), by
  equality with budget_select at its own B, and by the edge readings.
* uniform_k_select — pinned by the FOS truncated-k table (tokens per computed
  position is its goodput for one request whose step cost grows with the
  positions computed), by exact-rational search, by equality with the budget
  for a single request, by the budget's score bounding it, and by the DSD
  page's claim that the chosen K falls as the batch grows into the compute
  bound.
* accept_stats — pinned by a hand-derived case and by the FOS per-position
  table (conditional column = accepted / verified, cumulative = running
  product, mean acceptance length = 1 + sum of the cumulative column).
* draft_features (entropy in bits and largest probability of a draft row) —
  pinned by closed forms on uniform, k-point and two-point rows, by scipy's
  entropy and softmax on random rows, and by invariants (logit shift,
  temperature folded into the logits, min-entropy and support bounds,
  entropy rising with temperature).
* calibrate_update / calibrate_predict — pinned by finite differences of an
  independently written log-loss, by the gradient vanishing (in mean) at the
  parameters that generated the outcomes, by absent features reading as 0,
  and by the sign of an update.
* cost_table_prepare — pinned by the 121 -> 128 padding example on the
  agentlens page and by monotonicity.
* pack_varlen — pinned by hand-derived golden fixtures and capacity formula.
* verify (greedy) — pinned by a hand-derived golden fixture and by brute
  force per-row argmax.
* verify (stochastic) — pinned by exact enumeration of the output law on a
  32-token vocabulary (the law must equal the target distribution), by
  chi-square over seeded trials, by the closed form E[L] = sum_j prod_i alpha_i,
  and by the identity residual mass = 1 - sum min(p, q) = 0.5 * |p - q|_1.
"""

from .philox import philox4x32_10, uniforms, PHILOX_ROUNDS
from .budget import (
    clamp_confidence,
    survival,
    cost_table_prepare,
    rank_slots,
    fixed_point,
    expected_tokens,
    budget_score,
    budget_select,
    budget_allocate,
    DEV_BAD_DRAFT_LEN,
    DEV_BAD_COST,
)
from .uniform_k import uniform_k_select
from .calibrate import accept_stats, calibrate_update, predict as calibrate_predict
from .features import draft_features
from .pack import pack_varlen, DEV_BAD_KEPT
from .verify import (
    row_probs,
    accept,
    residual_weights,
    inverse_cdf,
    row_is_faulty,
    verify_request,
    verify,
    GREEDY,
    STOCHASTIC,
    DEV_BAD_CU_ROWS,
    DEV_BAD_TOKEN,
    DEV_NONFINITE,
)

__all__ = [
    "philox4x32_10", "uniforms", "PHILOX_ROUNDS",
    "clamp_confidence", "survival", "cost_table_prepare", "rank_slots",
    "fixed_point", "expected_tokens", "budget_score", "budget_select", "budget_allocate", "uniform_k_select",
    "accept_stats", "calibrate_update", "calibrate_predict", "draft_features",
    "pack_varlen", "row_probs", "accept", "residual_weights", "inverse_cdf",
    "row_is_faulty", "verify_request", "verify", "GREEDY", "STOCHASTIC",
    "DEV_BAD_DRAFT_LEN", "DEV_BAD_COST", "DEV_BAD_KEPT", "DEV_BAD_CU_ROWS",
    "DEV_BAD_TOKEN", "DEV_NONFINITE",
]
