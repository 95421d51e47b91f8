"""GPU (HIP, through the C ABI) versus the oracle, on seeded synthetic inputs.

Sizes: the five workloads at their real shapes (tiny, 16 x V32000,
64 x V128256, 256 x V129280, 256 x mixed K up to 15 x V256000), plus ragged
vocabularies, unaligned strides, several pass-2 tiles and the degenerate
cases (no drafts, empty batch, faults, masked logits, the exact fallback).
The comparison rules are in tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

from parity import (H_ATOL, H_RTOL, P_RTOL, check_allocate, check_budget, check_pack,
                    check_uniform_k,
                    compare_verify, gpu_verify, logits_dtype, to_dev, workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import adaptive_draft_verification_amd  # noqa: F401  (fails loudly if the library is missing)


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ Philox

def test_philox_bit_equal_to_oracle():
    import adaptive_draft_verification_amd as sv
    for seed, step, n, npos in [(0, 0, 256, 16), (2**63 + 12345, 2**40 + 7, 300, 65),
                                (123, 5, 4096, 8)]:
        u = torch.empty(n, npos, dtype=torch.float32, device="cuda")
        v = torch.empty_like(u)
        sv.sv_philox_uniforms(seed, step, u, v)
        torch.cuda.synchronize()
        r = np.repeat(np.arange(n), npos)
        j = np.tile(np.arange(npos), n)
        ou, ov = oracle.uniforms(seed, r, j, step)
        np.testing.assert_array_equal(u.cpu().numpy().ravel(), ou.astype(np.float32))
        np.testing.assert_array_equal(v.cpu().numpy().ravel(), ov.astype(np.float32))


# ------------------------------------------------------------------ budget

@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_budget_workloads(name):
    w = workloads.make(name)
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    o = check_budget(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    log(f"{name}: B={o['budget']} kept rows={int(o['kept'].sum()) + w.n}")


@pytest.mark.parametrize("seed", range(40))
def test_budget_random(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(16, 8192 // n) + 1))
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(
        rng, n, k, ties=seed % 2 == 0, zeros=seed % 3 == 0, flat_cost=seed % 7 == 0)
    if seed % 5 == 0:
        cost = np.maximum.accumulate(cost)
    if seed % 11 == 0:  # out-of-range draft lengths and bad confidences
        dl[0] = k + 3
        dl[-1] = -2
        conf[0, 0] = np.nan
        conf[-1, -1] = 7.0
    if seed % 13 == 0:  # some unusable cost entries
        cost[t_base + 1] = np.nan
        cost[-1] = 0.0
    check_budget(conf, dl, k, cost, t_base, n_bonus)


@pytest.mark.parametrize("n,k", [(8192, 1), (1024, 8), (512, 16), (128, 64), (1, 1), (3, 0),
                                 (0, 4)])
def test_budget_edges(n, k):
    rng = np.random.default_rng(n + k)
    conf = rng.uniform(0.3, 1.0, (n, k)).astype(np.float32)
    dl = rng.integers(0, k + 1, n).astype(np.int32)
    t = np.arange(n + n * k + 1, dtype=np.float32)
    cost = np.maximum(1.0, t / max(1, n)).astype(np.float32)
    check_budget(conf, dl, k, cost, n, n)


def test_budget_denormal_survivals():
    conf = np.full((4, 6), 2.0 ** -30, dtype=np.float32)
    conf[:, 0] = 0.5
    dl = np.full(4, 6, dtype=np.int32)
    cost = np.ones(4 + 24 + 1, dtype=np.float32)
    check_budget(conf, dl, 6, cost, 4, 4)


# ------------------------------------------- a budget sized from stale confidences

@pytest.mark.parametrize("seed", range(24))
def test_budget_allocate_random(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(16, 8192 // n) + 1))
    conf, dl, _cost, _t, _nb = workloads.random_budget_case(rng, n, k, ties=seed % 2 == 0,
                                                            zeros=seed % 3 == 0)
    if seed % 7 == 0:
        dl[0] = k + 2
        conf[-1, 0] = np.nan
    total = int(np.clip(dl, 0, k).sum())
    for B in (-3, 0, 1, int(rng.integers(0, total + 1)), total, total + 5):
        check_allocate(conf, dl, k, B)


@pytest.mark.parametrize("n,k", [(8192, 1), (1024, 8), (128, 64), (1, 1), (3, 0), (0, 4)])
def test_budget_allocate_edges(n, k):
    rng = np.random.default_rng(n * 3 + k)
    conf = rng.uniform(0.3, 1.0, (n, k)).astype(np.float32)
    dl = rng.integers(0, k + 1, n).astype(np.int32)
    for B in (0, n * k // 3, n * k):
        check_allocate(conf, dl, k, B)


def test_stale_budget_pipeline():
    """The agentlens Execution Pipeline on one stream: step t's budget is sized
    from step t-1's confidences (double-buffered on the device) and reaches the
    host through an asynchronous copy into pinned memory; the slots come from
    step t's confidences on the device; pack and verify follow.  Each stage
    against the oracle fed the same inputs."""
    import adaptive_draft_verification_amd as sv
    w = workloads.make("b64_v128256")
    n, k = w.n, w.k_max
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    rng = np.random.default_rng(3)
    steps = 4
    confs = [w.conf] + [(rng.beta(8, 2, (n, 1)) ** np.arange(1, k + 1)).astype(np.float32)
                        for _ in range(steps - 1)]
    conf_buf = [torch.empty(n, k, dtype=torch.float32, device="cuda") for _ in range(2)]
    dl, cost_d = to_dev(w.draft_len), to_dev(cost)
    toks = w.draft_tokens("stochastic")
    budget_dev = torch.empty(1, dtype=torch.int32, device="cuda")
    kept_sel = torch.empty(n, dtype=torch.int32, device="cuda")
    b_host = torch.empty(1, dtype=torch.int32).pin_memory()
    copied = torch.cuda.Event()
    ws = torch.empty(sv.sv_budget_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    draft_full = workloads.assemble_draft(w, w.draft_len)
    for t in range(steps):
        cur = conf_buf[t % 2]
        cur.copy_(torch.from_numpy(confs[t]))            # the drafter's estimates of step t
        prev = conf_buf[(t - 1) % 2] if t > 0 else cur  # step 0 has no previous step
        prev_np = confs[t - 1] if t > 0 else confs[0]
        sv.sv_budget_select(prev, dl, cost_d, w.t_base, w.n_bonus, kept_sel, budget_dev, ws=ws)
        b_host.copy_(budget_dev, non_blocking=True)
        copied.record()
        copied.synchronize()                             # the scheduler sizes the batch
        B = int(b_host[0])
        assert B == oracle.budget_select(prev_np, w.draft_len, k, cost, w.t_base,
                                         w.n_bonus)["budget"]
        a = sv.budget_allocate(cur, dl, budget_dev, ws=ws)
        p = sv.pack_varlen(a["kept"], to_dev(w.last_token), to_dev(toks))
        o_a = oracle.budget_allocate(confs[t], w.draft_len, k, B)
        np.testing.assert_array_equal(a["kept"].cpu().numpy(), o_a["kept"])
        kept = o_a["kept"]
        o_p = oracle.pack_varlen(kept, w.last_token, toks, k)
        np.testing.assert_array_equal(p["cu_rows"].cpu().numpy(), o_p["cu_rows"])
        target = workloads.assemble_target(w, o_p["cu_rows"], kept)
        v = sv.verify(to_dev(target, logits_dtype(w)), to_dev(draft_full, logits_dtype(w)),
                      to_dev(toks), p["cu_rows"], sv.SV_STOCHASTIC, w.tau, w.seed, t)
        torch.cuda.synchronize()
        g = {key: val.cpu().numpy() for key, val in v.items()}
        compare_verify(g, target, draft_full, toks, o_p["cu_rows"], k, w.vocab, "stochastic",
                       w.tau, w.seed, t)
        log(f"step {t}: B={B} rows={int(o_p['cu_rows'][-1])}")
    w.drop_cache()


def test_allocate_graph_replay_follows_the_budget_in_memory():
    """allocate -> pack captured once; replays read whatever B and confidences
    sit in their device buffers (written by kernels between replays)."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(12)
    n, k = 200, 7
    conf_np = [(rng.beta(8, 2, (n, 1)) ** np.arange(1, k + 1)).astype(np.float32)
               for _ in range(3)]
    dl_np = rng.integers(0, k + 1, n).astype(np.int32)
    conf, dl = torch.empty(n, k, dtype=torch.float32, device="cuda"), to_dev(dl_np)
    b_in = torch.zeros(1, dtype=torch.int32, device="cuda")
    last, toks = to_dev(rng.integers(0, 999, n).astype(np.int32)), \
        to_dev(rng.integers(0, 999, (n, k)).astype(np.int32))
    ws = torch.empty(sv.sv_budget_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    kept = torch.empty(n, dtype=torch.int32, device="cuda")
    used = torch.empty(1, dtype=torch.int32, device="cuda")
    cap = n * (k + 1)
    cu = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    rr, rp, pt = (torch.empty(cap, dtype=torch.int32, device="cuda") for _ in range(3))

    def body():
        sv.sv_budget_allocate(conf, dl, b_in, kept, used, ws=ws)
        sv.sv_pack_varlen(kept, last, toks, cu, rr, rp, pt)

    conf.copy_(torch.from_numpy(conf_np[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    total = int(np.clip(dl_np, 0, k).sum())
    for i, B in enumerate([0, 17, total // 2, total + 3, 5]):
        c = conf_np[i % 3]
        conf.copy_(torch.from_numpy(c))
        b_in.fill_(B)
        g.replay()
        torch.cuda.synchronize()
        o = oracle.budget_allocate(c, dl_np, k, B)
        np.testing.assert_array_equal(kept.cpu().numpy(), o["kept"], err_msg=f"replay {i}")
        assert int(used.cpu()[0]) == o["budget_used"]
        o_p = oracle.pack_varlen(o["kept"], last.cpu().numpy(), toks.cpu().numpy(), k)
        np.testing.assert_array_equal(cu.cpu().numpy(), o_p["cu_rows"], err_msg=f"replay {i}")
        body()  # eager work between replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kept.cpu().numpy(), o["kept"])


# ------------------------------------------ budget and pack in one launch fewer

def check_fused_pack(conf, dl, k, cost=None, t_base=0, n_bonus=0, budget=None, seed=0):
    """sv_budget_select_pack (cost given) or sv_budget_allocate_pack (budget
    given) against the oracle's budget and pack, every output bit for bit."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(seed)
    n = len(dl)
    last = rng.integers(0, 50000, n).astype(np.int32)
    toks = rng.integers(0, 50000, (n, k)).astype(np.int32)
    cap = n * (k + 1)
    kept = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    b = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    surv = torch.empty(n, k, dtype=torch.float32, device="cuda")
    cu = torch.full((n + 1,), -7, dtype=torch.int32, device="cuda")
    rr, rp, pt = (torch.full((cap,), -7, dtype=torch.int32, device="cuda") for _ in range(3))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, sv.sv_budget_workspace_bytes(n, k)), dtype=torch.uint8,
                     device="cuda")
    args = (to_dev(last), to_dev(toks))
    if budget is None:
        sv.sv_budget_select_pack(to_dev(conf), to_dev(dl), to_dev(cost), t_base, n_bonus, *args,
                                 kept, b, cu, rr, rp, pt, surv, err, ws=ws)
        o = oracle.budget_select(conf, dl, k, cost, t_base, n_bonus)
        want_b = o["budget"]
    else:
        sv.sv_budget_allocate_pack(to_dev(conf), to_dev(dl), to_dev(np.array([budget], np.int32)),
                                   *args, kept, cu, rr, rp, pt, b, surv, err, ws=ws)
        o = oracle.budget_allocate(conf, dl, k, budget)
        want_b = o["budget_used"]
    torch.cuda.synchronize()
    op = oracle.pack_varlen(o["kept"], last, toks, k)
    np.testing.assert_array_equal(kept.cpu().numpy(), o["kept"])
    assert int(b.cpu()[0]) == want_b
    np.testing.assert_array_equal(surv.cpu().numpy().view(np.uint32), o["survival"].view(np.uint32))
    for key, t in (("cu_rows", cu), ("row_req", rr), ("row_pos", rp), ("packed_tokens", pt)):
        np.testing.assert_array_equal(t.cpu().numpy(), op[key], err_msg=key)
    assert int(err.cpu()[0]) == o["dev_error"] | op["dev_error"]


@pytest.mark.parametrize("seed", range(16))
def test_budget_select_pack_random(seed):
    rng = np.random.default_rng(900 + seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(16, 8192 // n) + 1))
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(
        rng, n, k, ties=seed % 2 == 0, zeros=seed % 3 == 0, flat_cost=seed % 5 == 0)
    if seed % 7 == 0:
        dl[0] = k + 3
        dl[-1] = -1
    check_fused_pack(conf, dl, k, cost, t_base, n_bonus, seed=seed)
    total = int(np.clip(dl, 0, k).sum())
    for B in (-2, 0, total // 3, total + 4):
        check_fused_pack(conf, dl, k, budget=B, seed=seed)


@pytest.mark.parametrize("n,k", [(8192, 1), (1024, 8), (128, 64), (4096, 2), (1, 1), (3, 0),
                                 (0, 4)])
def test_budget_pack_fused_edges(n, k):
    rng = np.random.default_rng(n + 7 * k)
    conf = rng.uniform(0.3, 1.0, (n, k)).astype(np.float32)
    dl = rng.integers(0, k + 1, n).astype(np.int32)
    t = np.arange(n + n * k + 1, dtype=np.float32)
    cost = np.maximum(1.0, t / max(1, n)).astype(np.float32)
    check_fused_pack(conf, dl, k, cost, n, n)
    check_fused_pack(conf, dl, k, budget=n * k // 2)


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_budget_select_pack_workloads(name):
    w = workloads.make(name)
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    check_fused_pack(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)


# ------------------------------------------------------- uniform draft length

@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_uniform_k_workloads(name):
    w = workloads.make(name)
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    o = check_uniform_k(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    log(f"{name}: K*={o['k']}")


@pytest.mark.parametrize("seed", range(30))
def test_uniform_k_random(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(16, 8192 // n) + 1))
    conf, dl, cost, t_base, n_bonus = workloads.random_budget_case(
        rng, n, k, ties=seed % 2 == 0, zeros=seed % 3 == 0, flat_cost=seed % 7 == 0)
    if seed % 5 == 0:
        cost = np.maximum.accumulate(cost)
    if seed % 11 == 0:
        dl[0] = k + 3
        dl[-1] = -2
        conf[0, 0] = np.nan
    if seed % 13 == 0:
        cost[t_base + 1] = np.nan
    check_uniform_k(conf, dl, k, cost, t_base, n_bonus)


@pytest.mark.parametrize("n,k", [(8192, 1), (1024, 8), (128, 64), (1, 64), (1, 1), (3, 0),
                                 (0, 4)])
def test_uniform_k_edges(n, k):
    rng = np.random.default_rng(n + 3 * k)
    conf = rng.uniform(0.3, 1.0, (n, k)).astype(np.float32)
    dl = rng.integers(0, k + 1, n).astype(np.int32)
    t = np.arange(n + n * k + 1, dtype=np.float32)
    cost = np.maximum(1.0, t / max(1, n)).astype(np.float32)
    check_uniform_k(conf, dl, k, cost, n, n)


# -------------------------------------------------------------------- pack

@pytest.mark.parametrize("seed", range(12))
def test_pack_random(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 3000))
    k = int(rng.integers(0, 16))
    kept = rng.integers(0, k + 1, n)
    if seed % 4 == 0 and n:
        kept[0] = k + 5  # clamped, flagged
        kept[-1] = -1
    check_pack(kept, rng.integers(0, 1000, n), rng.integers(0, 1000, (n, k)), k)


# ------------------------------------------------------------------ verify

def run_workload_verify(name, mode, adaptive, features=False):
    w = workloads.make(name)
    if adaptive:
        cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
        kept = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base,
                                    w.n_bonus)["kept"]
    else:
        kept = w.draft_len.copy()
    target, draft, toks, cu = workload_inputs(w, kept, mode)
    log(f"{name} {mode} adaptive={adaptive} features={features}: rows={int(cu[-1])} "
        f"V={w.vocab}")
    g = gpu_verify(target, draft, toks, cu, w.k_max, mode, w.tau, logits_dtype(w),
                   seed=w.seed, step=w.step, features=features)
    stats = compare_verify(g, target, draft, toks, cu, w.k_max, w.vocab, mode, w.tau, w.seed,
                           w.step)
    log(f"  {stats}")
    w.drop_cache()
    return g, stats


@pytest.mark.parametrize("features", [False, True])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
@pytest.mark.parametrize("name,adaptive", [("tiny", True), ("tiny", False),
                                           ("b16_v32000", False), ("b64_v128256", True)])
def test_verify_small_workloads(name, adaptive, mode, features):
    run_workload_verify(name, mode, adaptive, features)


@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_verify_b64_full_k(mode):
    run_workload_verify("b64_v128256", mode, False)


@pytest.mark.parametrize("adaptive", [True, False])
def test_verify_b256_v129280_stochastic(adaptive):
    g, stats = run_workload_verify("b256_v129280", "stochastic", adaptive)
    assert stats["u_band"] + stats["cdf_band"] <= 3


def test_verify_b256_v129280_greedy():
    run_workload_verify("b256_v129280", "greedy", False)


def test_verify_b256_mix_v256000():
    run_workload_verify("b256_mix_v256000", "stochastic", True, features=True)


def test_features_leave_the_decisions_alone():
    """Asking for the draft-row features switches pass 1's draft rows to the
    accumulating kernel; the row statistics, hence every decision, draw and
    probability, must come out bit for bit as without it."""
    w = workloads.make("b256_v129280")
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    kept = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)["kept"]
    target, draft, toks, cu = workload_inputs(w, kept, "stochastic")
    a = gpu_verify(target, draft, toks, cu, w.k_max, "stochastic", w.tau, logits_dtype(w),
                   seed=w.seed, step=w.step)
    b = gpu_verify(target, draft, toks, cu, w.k_max, "stochastic", w.tau, logits_dtype(w),
                   seed=w.seed, step=w.step, features=True)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    # features at sampled kept positions against the oracle
    rng = np.random.default_rng(0)
    for r in rng.choice(w.n, 12, replace=False):
        for j in range(int(kept[r])):
            h, m = oracle.draft_features(draft[r * w.k_max + j, : w.vocab], w.tau)
            assert abs(b["q_entropy"][r, j] - h) <= H_ATOL + H_RTOL * h, (r, j)
            assert abs(b["q_max"][r, j] - m) <= P_RTOL * m, (r, j)
    w.drop_cache()


# ------------------------------------------------------- shapes and edge cases

def synthetic(rng, n, k, V, kept=None, scale=3.0):
    kept = rng.integers(0, k + 1, n) if kept is None else np.asarray(kept)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    target = (rng.standard_normal((int(cu[-1]), V)) * scale).astype(np.float32)
    draft = np.full((n * k, V), np.nan, dtype=np.float32)
    toks = np.full((n, k), -1, dtype=np.int32)
    for r in range(n):
        for j in range(int(kept[r])):
            row = target[cu[r] + j] + rng.standard_normal(V).astype(np.float32)
            draft[r * k + j] = row
            toks[r, j] = int(np.argmax(row - np.log(rng.standard_exponential(V))))
    return target, draft, toks, cu


def bf16_round(a):
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("dtype,V,ld_pad,tau", [
    (torch.bfloat16, 129280, 0, 1.0),
    (torch.bfloat16, 131072, 0, 0.5),   # the largest one-part row
    (torch.bfloat16, 8193, 0, 1.8),     # a ragged scalar tail
    (torch.bfloat16, 4100, 0, 1.0),     # a few bonus super-groups
    (torch.float32, 100003, 0, 0.7),
    (torch.float32, 65536, 2, 1.0),     # rows off 16-byte alignment
    (torch.float32, 131073, 0, 1.0),    # two row parts
])
def test_verify_bonus_draws(dtype, V, ld_pad, tau):
    """Every draft accepted (each draft row equals its target row, so p/q = 1):
    every request's token is a bonus draw from target row b (FOS "평균 수락 길이":
    the token the target picks itself after the last accepted draft)."""
    rng = np.random.default_rng(V + ld_pad)
    n, k = 96, 3
    kept = rng.integers(0, k + 1, n)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    target = (rng.standard_normal((int(cu[-1]), V)) * 3).astype(np.float32)
    if dtype == torch.bfloat16:
        target = bf16_round(target)
    draft = np.full((n * k, V), np.nan, dtype=np.float32)
    toks = np.full((n, k), -1, dtype=np.int32)
    for r in range(n):
        for j in range(int(kept[r])):
            row = target[cu[r] + j]
            draft[r * k + j] = row
            toks[r, j] = int(np.argmax(row / tau - np.log(rng.standard_exponential(V))))
    log(f"bonus draws: {dtype} V={V} ld_pad={ld_pad} tau={tau}")
    g = gpu_verify(target, draft, toks, cu, k, "stochastic", tau, dtype, seed=V, step=3,
                   target_ld=V + ld_pad, draft_ld=V + ld_pad)
    np.testing.assert_array_equal(g["accepted"], kept)
    stats = compare_verify(g, target, draft, toks, cu, k, V, "stochastic", tau, seed=V, step=3)
    log(f"  {stats}")
    # A bonus draw stops its sweep once the summed super-groups pass v * W,
    # which happens at a time that varies from call to call; the drawn ids
    # must not: repeated calls agree bit for bit.
    for _ in range(8):
        again = gpu_verify(target, draft, toks, cu, k, "stochastic", tau, dtype, seed=V, step=3,
                           target_ld=V + ld_pad, draft_ld=V + ld_pad)
        for key in ("tokens", "accepted", "p_draft", "q_draft", "residual_mass"):
            np.testing.assert_array_equal(again[key], g[key], err_msg=key)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,ld_pad", [(1003, 0), (20001, 0), (32, 3), (8192 * 3 + 5, 1),
                                      (1, 0), (7, 0), (131073, 1), (400003, 0)])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_verify_ragged_vocab_and_strides(dtype, V, ld_pad, mode):
    rng = np.random.default_rng(V + ld_pad)
    n, k = 9, 4
    target, draft, toks, cu = synthetic(rng, n, k, V)
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"ragged V={V} ld_pad={ld_pad} {dtype} {mode}")
    g = gpu_verify(target, draft if mode == "stochastic" else None, toks, cu, k, mode, 0.8,
                   dtype, seed=3, step=11, target_ld=V + ld_pad, draft_ld=V + ld_pad,
                   features=True)
    compare_verify(g, target, draft if mode == "stochastic" else None, toks, cu, k, V, mode, 0.8,
                   3, 11)


@pytest.mark.parametrize("seed", list(range(16)) + [41, 48, 59, 84, 119, 151, 172, 194, 228])
def test_verify_random_shapes(seed):
    """Seeded random shapes: batch, draft count, vocabulary (one super-group
    to several row parts' worth of groups), row stride, dtype, mode,
    temperature, Philox step and kept counts, each against the oracle.
    Seeds 41 to 228 draw peaked rows (logit scale 8, or T = 0.3) with small
    residual masses, which exponents rounded far from the row's peak once
    put outside the residual-mass tolerance."""
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 25))
    k = int(rng.integers(0, 10))
    V = int(rng.choice([int(rng.integers(1, 600)), int(rng.integers(600, 20000)),
                        int(rng.integers(20000, 70000))]))
    ld_pad = int(rng.integers(0, 4))
    dtype = torch.bfloat16 if seed % 2 == 0 else torch.float32
    mode = "greedy" if seed % 5 == 0 else "stochastic"
    tau = float(rng.choice([0.3, 0.7, 1.0, 1.8]))
    step = int(rng.integers(0, 2 ** 40))
    target, draft, toks, cu = synthetic(rng, n, k, V, scale=float(rng.choice([1.0, 3.0, 8.0])))
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"random shapes seed={seed}: n={n} k={k} V={V} ld_pad={ld_pad} {dtype} {mode} "
        f"tau={tau} step={step}")
    dmode = draft if mode == "stochastic" else None
    g = gpu_verify(target, dmode, toks, cu, k, mode, tau, dtype, seed=seed, step=step,
                   target_ld=V + ld_pad, draft_ld=V + ld_pad, features=seed % 3 == 0)
    compare_verify(g, target, dmode, toks, cu, k, V, mode, tau, seed, step)


@pytest.mark.parametrize("seed", range(8))
def test_verify_random_large_vocab(seed):
    """Seeded random batches at vocabularies of 100,000 to SV_MAX_VOCAB ids
    (two to eight row parts whose offsets and sums merge in pass 2), both
    dtypes, peaked and flat rows; every other case accepts every draft, so
    its tokens are bonus draws whose sweeps stop early."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(60000 + seed)
    n = int(rng.integers(1, 6))
    k = int(rng.integers(1, 8))
    V = int(rng.choice([int(rng.integers(100000, 300000)),
                        int(rng.integers(300000, sv.SV_MAX_VOCAB + 1))]))
    dtype = torch.bfloat16 if seed % 2 == 0 else torch.float32
    mode = "greedy" if seed == 7 else "stochastic"
    tau = float(rng.choice([0.3, 0.7, 1.0, 1.8]))
    step = int(rng.integers(0, 2 ** 40))
    ld_pad = int(rng.integers(0, 3))
    target, draft, toks, cu = synthetic(rng, n, k, V, scale=float(rng.choice([1.0, 3.0, 8.0])))
    if seed % 2 == 1:
        for r in range(n):
            for j in range(int(cu[r + 1] - cu[r] - 1)):
                draft[r * k + j] = target[cu[r] + j]
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"large vocab seed={seed}: n={n} k={k} V={V} {dtype} {mode} tau={tau}")
    dmode = draft if mode == "stochastic" else None
    g = gpu_verify(target, dmode, toks, cu, k, mode, tau, dtype, seed=seed, step=step,
                   target_ld=V + ld_pad, draft_ld=V + ld_pad, features=seed % 3 == 0)
    compare_verify(g, target, dmode, toks, cu, k, V, mode, tau, seed, step)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
@pytest.mark.parametrize("which", ["vocab", "drafts"])
def test_verify_maximum_sizes(which, dtype, mode):
    """The largest vocabulary (SV_MAX_VOCAB: 8 row parts, the most super-
    groups per draw) and the largest draft count (SV_MAX_DRAFT: one wave64
    ballot per request), with a request that keeps every draft, one that keeps
    some and one that keeps none."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(2024)
    if which == "vocab":
        n, k, V, kept = 3, 3, sv.SV_MAX_VOCAB, [3, 1, 0]
    else:
        n, k, V, kept = 3, sv.SV_MAX_DRAFT, 20001, [sv.SV_MAX_DRAFT, 17, 0]
    target, draft, toks, cu = synthetic(rng, n, k, V, kept)
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"maximum {which}: V={V} k={k} {dtype} {mode}: rows={int(cu[-1])}")
    dmode = draft if mode == "stochastic" else None
    g = gpu_verify(target, dmode, toks, cu, k, mode, 1.0, dtype, seed=13, step=5, features=True)
    compare_verify(g, target, dmode, toks, cu, k, V, mode, 1.0, 13, 5)


@pytest.mark.parametrize("n", [512, 513])
def test_verify_dense_order_limit(n):
    """512 requests take the dense pass-1 order, 513 the per-request one."""
    rng = np.random.default_rng(n)
    k, V = 3, 3001
    target, draft, toks, cu = synthetic(rng, n, k, V)
    for mode in ("stochastic", "greedy"):
        dmode = draft if mode == "stochastic" else None
        g = gpu_verify(target, dmode, toks, cu, k, mode, 1.1, torch.bfloat16 if n == 512 else
                       torch.float32, seed=4, step=1, features=True)
        t = bf16_round(target) if n == 512 else target
        d = (bf16_round(draft) if n == 512 else draft) if dmode is not None else None
        compare_verify(g, t, d, toks, cu, k, V, mode, 1.1, 4, 1)


def test_verify_many_small_requests():
    rng = np.random.default_rng(77)
    n, k, V = 4096, 2, 1000
    target, draft, toks, cu = synthetic(rng, n, k, V)
    g = gpu_verify(target, draft, toks, cu, k, "stochastic", 0.9, torch.float32, seed=1, step=2,
                   features=True)
    compare_verify(g, target, draft, toks, cu, k, V, "stochastic", 0.9, 1, 2)


@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_verify_no_drafts(mode):
    rng = np.random.default_rng(5)
    n, V = 6, 4000
    target = (rng.standard_normal((n, V)) * 3).astype(np.float32)
    cu = np.arange(n + 1, dtype=np.int32)
    toks = np.zeros((n, 0), dtype=np.int32)
    draft = np.zeros((0, V), dtype=np.float32) if mode == "stochastic" else None
    g = gpu_verify(target, draft, toks, cu, 0, mode, 1.0, torch.float32, features=True)
    compare_verify(g, target, draft, toks, cu, 0, V, mode, 1.0)
    assert (g["accepted"] == 0).all()


def test_verify_empty_batch():
    import adaptive_draft_verification_amd as sv
    out = sv.verify(torch.zeros(1, 8, device="cuda"), torch.zeros(1, 8, device="cuda"),
                    torch.zeros(0, 2, dtype=torch.int32, device="cuda"),
                    torch.zeros(1, dtype=torch.int32, device="cuda"), sv.SV_STOCHASTIC)
    torch.cuda.synchronize()
    assert out["tokens"].numel() == 0 and int(out["dev_error"].item()) == 0


@pytest.mark.parametrize("mode", ["stochastic", "greedy"])
def test_verify_faults_and_masks(mode):
    rng = np.random.default_rng(17)
    n, k, V = 8, 3, 5000
    kept = np.array([3, 3, 3, 3, 2, 1, 0, 3])
    target, draft, toks, cu = synthetic(rng, n, k, V, kept)
    target[cu[1] + 1, 77] = np.nan                 # request 1: NaN in a target row
    toks[2, 1] = V + 4                             # request 2: draft id out of range
    draft[3 * k + 2, :] = -np.inf                  # request 3: draft row without mass
    target[cu[4] + 0, : V // 2] = -np.inf          # request 4: masked half row (legal)
    target[cu[5] + 1, 4000] = np.inf               # request 5: +inf logit
    target[cu[7] + 2, :] = -np.inf                 # request 7: target row without mass
    dmode = draft if mode == "stochastic" else None
    g = gpu_verify(target, dmode, toks, cu, k, mode, 1.0, torch.float32, features=True)
    compare_verify(g, target, dmode, toks, cu, k, V, mode, 1.0)
    assert g["accepted"][4] >= 0
    assert int(g["dev_error"][0]) != 0


def test_verify_bad_offsets_never_read_past_target_rows():
    rng = np.random.default_rng(23)
    n, k, V = 5, 2, 3000
    target, draft, toks, cu = synthetic(rng, n, k, V, [2, 2, 2, 2, 2])
    bad = cu.copy()
    bad[2] = bad[1] - 1       # request 1 negative length, request 2 too long
    bad[5] = bad[5] + 4       # request 4 runs past the buffer
    for mode in ("stochastic", "greedy"):
        dmode = draft if mode == "stochastic" else None
        g = gpu_verify(target, dmode, toks, bad, k, mode, 1.0, torch.float32, features=True)
        compare_verify(g, target, dmode, toks, bad, k, V, mode, 1.0)
        assert int(g["dev_error"][0]) & oracle.DEV_BAD_CU_ROWS


def test_verify_late_large_logit():
    """A logit far above the rest of its row, late in the row (the thread that
    meets it moves its offset by ~260 at once, its earlier sums scaling to
    nothing), one in a draft row, and a row whose logits drop by 120 after id
    5 (offsets set early lie far above the rest)."""
    rng = np.random.default_rng(29)
    n, k, V = 4, 2, 70000
    target, draft, toks, cu = synthetic(rng, n, k, V, [2, 2, 2, 2])
    target[cu[1] + 0, V - 3] = 180.0
    draft[2 * k + 1, 65000] = 150.0
    target[cu[3] + 2, 5:] -= 120.0
    for dtype in (torch.float32, torch.bfloat16):
        t = target if dtype == torch.float32 else bf16_round(target)
        d = draft if dtype == torch.float32 else bf16_round(draft)
        for features in (False, True):
            g = gpu_verify(t, d, toks, cu, k, "stochastic", 1.0, dtype, seed=9,
                           features=features)
            compare_verify(g, t, d, toks, cu, k, V, "stochastic", 1.0, 9)


def test_verify_low_temperature_and_ties():
    rng = np.random.default_rng(31)
    n, k, V = 16, 4, 9000
    target, draft, toks, cu = synthetic(rng, n, k, V)
    target = np.round(target)  # many exact ties
    draft = np.round(draft)
    for tau in (0.05, 3.0):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", tau, torch.float32, seed=2,
                       features=True)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", tau, 2)
    g = gpu_verify(target, None, toks, cu, k, "greedy", 1.0, torch.float32)
    compare_verify(g, target, None, toks, cu, k, V, "greedy", 1.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("tau", [0.5, 1.0])
def test_verify_rising_and_outlier_rows(dtype, tau):
    """Rows that move pass 1's per-thread offsets again and again: a steep
    ramp (every chunk of every thread enters far above the offset before it),
    ascending and descending sorted rows, and a single outlier far above the
    rest at the last id or at id 0 (the id holds nearly all of p).  The
    entropy and largest-probability features ride along, so their rescaling
    on each move is checked too."""
    rng = np.random.default_rng(97)
    n, k, V = 6, 3, 20001
    kept = np.full(n, k)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    rows = int(cu[-1])
    target = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    ids = np.arange(V, dtype=np.float32)
    for r in range(n):
        for j in range(k + 1):
            t = target[cu[r] + j]
            if r == 0:
                t[:] = ids * 0.01 - 100.0            # ramp from -100 to +100
            elif r == 1:
                t[:] = np.sort(t)                    # ascending
            elif r == 2:
                t[:] = np.sort(t)[::-1]              # descending
            elif r == 3:
                t[-1] = 60.0                         # outlier at the last id
            elif r == 4:
                t[0] = 60.0                          # outlier at id 0
            else:
                t[:] = -ids * 0.01 + 50.0            # falling ramp
    draft = np.full((n * k, V), np.nan, dtype=np.float32)
    toks = np.full((n, k), -1, dtype=np.int32)
    for r in range(n):
        for j in range(k):
            row = target[cu[r] + j] + rng.standard_normal(V).astype(np.float32)
            draft[r * k + j] = row
            toks[r, j] = int(np.argmax(row / tau - np.log(rng.standard_exponential(V))))
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"rising and outlier rows: {dtype} tau={tau}")
    for step in range(3):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", tau, dtype, seed=4, step=step,
                       features=True)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", tau, 4, step)


def test_verify_draw_lands_on_positive_weight():
    """Residuals with zero weight on every other id, drawn many times: every
    drawn id must carry weight (the oracle's rule never lands on a zero)."""
    rng = np.random.default_rng(41)
    n, k, V = 64, 1, 40000
    target = (rng.standard_normal((2 * n, V)) * 2).astype(np.float32)
    cu = np.arange(0, 2 * n + 1, 2, dtype=np.int32)
    draft = target[0::2].copy()
    draft[:, 1::2] += 3.0  # q > p on odd ids: zero residual weight there
    toks = np.ones((n, k), dtype=np.int32)  # an odd id: mostly rejected
    for step in range(6):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", 1.0, torch.float32, seed=5,
                       step=step)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", 1.0, 5, step)
        rej = g["accepted"] == 0
        assert rej.sum() > n // 4
        assert (g["tokens"][rej, 0] % 2 == 0).all()


def _far_rows(rng, n, k, V, center, spread, masked, tau):
    """n requests at full K whose target and draft rows are center + spread * N(0, 1),
    the first `masked` ids of every row -inf; draft ids drawn from the draft rows at tau."""
    kept = np.full(n, k)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    target = (center + spread * rng.standard_normal((int(cu[-1]), V))).astype(np.float32)
    target[:, :masked] = -np.inf
    draft = np.empty((n * k, V), dtype=np.float32)
    toks = np.empty((n, k), dtype=np.int32)
    for r in range(n):
        for j in range(k):
            row = target[cu[r] + j] + (0.3 * spread * rng.standard_normal(V)).astype(np.float32)
            draft[r * k + j] = row
            toks[r, j] = int(np.argmax(row / tau - np.log(rng.standard_exponential(V))))
    return target, draft, toks, cu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,center,spread,masked,tau", [
    (5000, -86.0, 1.0, 2048, 1.0),      # masked prefix, mass near 2^-124
    (3000, -88.0, 1.0, 0, 1.0),         # short row: threads without ids
    (1003, -88.0, 1.0, 0, 1.0),
    (4095, -86.0, 1.0, 0, 1.0),
    (5000, -4.3, 0.05, 2048, 0.05),     # the same scale reached through a low temperature
    (129280, -86.0, 1.0, 4096, 1.0),    # every thread's first chunk masked
    (200003, -87.0, 1.0, 3000, 1.0),    # two row parts
])
def test_verify_far_negative_logits(dtype, V, center, spread, masked, tau):
    """Rows whose whole mass lies near the bottom of fp32's normal range, with and
    without a masked prefix: threads that meet no finite logit first, or no id at
    all, must not move the row's offset, and no term may flush (each thread takes
    its terms within a few units of its own largest logit)."""
    rng = np.random.default_rng(V + masked)
    n, k = 4, 3
    target, draft, toks, cu = _far_rows(rng, n, k, V, center, spread, masked, tau)
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    log(f"far-negative V={V} center={center} masked={masked} tau={tau} {dtype}")
    for features in (False, True):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", tau, dtype, seed=4,
                       features=features)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", tau, 4)
        assert int(g["dev_error"][0]) == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_finite_mask_far_below_the_row(dtype):
    """Ids masked with a finite logit (-88) in every first chunk of half the
    threads, whose later ids sit 9 below the rest: those threads first take an
    offset more than 126 (log2 units) below the row's and then move it, and their
    sums, large in their own scale, must survive the moves and the merges (a
    rescale that flushed below 2^-126 would drop ~1e-4 of the mass)."""
    E = 8 if dtype == torch.bfloat16 else 4
    rng = np.random.default_rng(61)
    n, k, V = 3, 2, 6144
    ids = np.arange(V)
    base = np.where(((ids // E) % 512) < 256, -9.0, 0.0)
    kept = np.full(n, k)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    target = (base + 0.1 * rng.standard_normal((int(cu[-1]), V))).astype(np.float32)
    target[:, : 256 * E] = -88.0
    draft = (target[np.repeat(np.arange(n) * (k + 1), k) + np.tile(np.arange(k), n)]
             + 0.05 * rng.standard_normal((n * k, V))).astype(np.float32)
    draft[:, : 256 * E] = -88.0
    toks = rng.integers(256 * E, V, (n, k)).astype(np.int32)
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    for features in (False, True):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", 1.0, dtype, seed=6,
                       features=features)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", 1.0, 6)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_zero_draft_probability(dtype):
    """q(d) = 0 (a -inf draft logit at the draft id): accepted whenever p(d) > 0,
    rejected when p(d) = 0 too (then the residual is drawn), whatever u.  Ids in
    the first and the second row part and in the ragged tail (V = 200003: two
    parts, V not a multiple of 8)."""
    rng = np.random.default_rng(67)
    n, k, V = 6, 3, 200003
    target, draft, toks, cu = synthetic(rng, n, k, V, np.full(n, k))
    tail, second, first = V - 1, 150001, 7

    def q_zero(r, j, d, p_zero=False):
        toks[r, j] = d
        draft[r * k + j, d] = -np.inf
        if p_zero:
            target[cu[r] + j, d] = -np.inf

    q_zero(0, 0, second)                 # accept at 0
    q_zero(1, 0, first)
    q_zero(1, 1, tail)                   # accept at 0 and 1
    q_zero(2, 0, second, p_zero=True)    # reject at 0
    q_zero(3, 0, tail)
    q_zero(3, 1, first)
    q_zero(3, 2, tail - 1, p_zero=True)  # accept 0, 1; reject at 2
    q_zero(4, 0, first, p_zero=True)     # reject at 0
    if dtype == torch.bfloat16:
        target, draft = bf16_round(target), bf16_round(draft)
    for seed in range(3):
        g = gpu_verify(target, draft, toks, cu, k, "stochastic", 0.9, dtype, seed=seed,
                       features=True)
        compare_verify(g, target, draft, toks, cu, k, V, "stochastic", 0.9, seed)
        acc = g["accepted"]
        assert acc[0] >= 1 and acc[1] >= 2 and acc[2] == 0 and acc[3] == 2 and acc[4] == 0
        assert g["q_draft"][0, 0] == 0 and g["p_draft"][0, 0] > 0
        assert g["q_draft"][2, 0] == 0 and g["p_draft"][2, 0] == 0
        assert g["tokens"][2, 0] != second and g["tokens"][4, 0] != first
        assert g["tokens"][3, 2] != tail - 1


def test_verify_is_deterministic_and_stream_safe():
    rng = np.random.default_rng(37)
    n, k, V = 32, 7, 50000
    target, draft, toks, cu = synthetic(rng, n, k, V)
    a = gpu_verify(target, draft, toks, cu, k, "stochastic", 1.0, torch.bfloat16, seed=4, step=2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_verify(target, draft, toks, cu, k, "stochastic", 1.0, torch.bfloat16, seed=4,
                       step=2)
    torch.cuda.synchronize()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = gpu_verify(target, draft, toks, cu, k, "stochastic", 1.0, torch.bfloat16, seed=4, step=3)
    assert not np.array_equal(a["tokens"], c["tokens"])


def test_concurrent_calls_on_two_streams():
    """Two different batches verified (and budgeted) at the same time on two
    streams, each call with its own workspace: every output equals the same
    call run alone (no state shared between calls outside the arguments)."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(53)
    cases = []
    for n, k, V, dtype in ((24, 5, 30011, torch.bfloat16), (17, 3, 12007, torch.float32)):
        target, draft, toks, cu = synthetic(rng, n, k, V)
        conf = rng.uniform(0.2, 1.0, (n, k)).astype(np.float32)
        dl = rng.integers(0, k + 1, n).astype(np.int32)
        cost = np.maximum(1.0, np.arange(n + n * k + 1) / 8.0).astype(np.float32)
        cases.append(dict(t=to_dev(target, dtype), d=to_dev(draft, dtype),
                          toks=to_dev(np.asarray(toks, np.int32)),
                          cu=to_dev(np.asarray(cu, np.int32)), conf=to_dev(conf), dl=to_dev(dl),
                          cost=to_dev(cost), n=n))

    def run(c, stream):
        v = sv.verify(c["t"], c["d"], c["toks"], c["cu"], sv.SV_STOCHASTIC, 0.9, 3, 8,
                      stream=stream)
        b = sv.budget_select(c["conf"], c["dl"], c["cost"], c["n"], c["n"], stream=stream)
        return v, b

    ref = [run(c, None) for c in cases]
    torch.cuda.synchronize()
    ref = [({k: x.cpu() for k, x in v.items()}, {k: x.cpu() for k, x in b.items()})
           for v, b in ref]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):  # enqueued back to back on both streams, no wait in between
        with torch.cuda.stream(s1):
            o1 = run(cases[0], s1)
        with torch.cuda.stream(s2):
            o2 = run(cases[1], s2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        for (v, b), (rv, rb) in zip((o1, o2), ref):
            for key in rv:
                assert torch.equal(v[key].cpu(), rv[key]), key
            for key in rb:
                assert torch.equal(b[key].cpu(), rb[key]), key


def test_debug_environment_variables(monkeypatch):
    """SV_DEBUG_CHECKS=1 refuses, on the host and before any launch, index data
    the kernels would flag in dev_error (SV_ERR_DATA; no output touched), and
    leaves good calls' results as they are; SV_FORCE_SYNC=1 changes no result.
    Under graph capture both are skipped, and the recorded call replays."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(77)
    n, k, V = 12, 3, 4099
    kept = np.array([3, 0, 2, 1, 3, 3, 0, 1, 2, 3, 1, 2])
    target, draft, toks, cu = synthetic(rng, n, k, V, kept=kept)
    t, d = to_dev(target), to_dev(draft)
    toks_d, cu_d = to_dev(np.asarray(toks, np.int32)), to_dev(np.asarray(cu, np.int32))
    ref = sv.verify(t, d, toks_d, cu_d, sv.SV_STOCHASTIC, 0.8, 5, 9)
    monkeypatch.setenv("SV_DEBUG_CHECKS", "1")
    monkeypatch.setenv("SV_FORCE_SYNC", "1")
    got = sv.verify(t, d, toks_d, cu_d, sv.SV_STOCHASTIC, 0.8, 5, 9)
    torch.cuda.synchronize()
    for key in ref:
        np.testing.assert_array_equal(ref[key].cpu().numpy(), got[key].cpu().numpy(), key)

    def refused(fn):
        with pytest.raises(sv.SvError) as e:
            fn()
        assert e.value.status == sv.SV_ERR_DATA, e.value

    outs = {key: torch.full_like(v, -5) for key, v in ref.items()}
    ws = torch.zeros(sv.sv_verify_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")

    def call(cu_x, toks_x):
        sv.sv_verify(t, d, toks_x, cu_x, sv.SV_STOCHASTIC, 0.8, 5, 9, outs["tokens"],
                     outs["accepted"], ws, outs["p_draft"], outs["q_draft"],
                     outs["residual_mass"], outs["dev_error"])

    bad_cu = np.asarray(cu, np.int32).copy()
    bad_cu[4] = bad_cu[3] - 1                       # request 3: negative row count
    refused(lambda: call(to_dev(bad_cu), toks_d))
    long_cu = np.asarray(cu, np.int32).copy()
    long_cu[1:] += 1                                 # request 0: k + 1 drafts
    refused(lambda: call(to_dev(long_cu), toks_d))
    bad_toks = np.asarray(toks, np.int32).copy()
    bad_toks[4, 2] = V                               # a kept draft id past the vocabulary
    refused(lambda: call(cu_d, to_dev(bad_toks)))
    unkept = np.asarray(toks, np.int32).copy()
    unkept[1, 0] = -9                                # request 1 keeps nothing: not looked at
    call(cu_d, to_dev(unkept))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs["tokens"].cpu().numpy(), ref["tokens"].cpu().numpy())
    for key, v in outs.items():
        v.fill_(-5)
    refused(lambda: call(to_dev(bad_cu), toks_d))
    torch.cuda.synchronize()
    assert (outs["tokens"] == -5).all() and (outs["accepted"] == -5).all()

    # the budget's draft lengths and the pack's kept counts
    conf = to_dev(rng.uniform(0.1, 1.0, (n, k)).astype(np.float32))
    cost = to_dev(np.linspace(1.0, 2.0, n * k + 1 + n).astype(np.float32))
    kept_o = torch.empty(n, dtype=torch.int32, device="cuda")
    budget = torch.empty(1, dtype=torch.int32, device="cuda")
    bws = torch.zeros(sv.sv_budget_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    dl = np.full(n, k, np.int32)
    sv.sv_budget_select(conf, to_dev(dl), cost, n, n, kept_o, budget, ws=bws)
    dl_bad = dl.copy()
    dl_bad[7] = k + 1
    refused(lambda: sv.sv_budget_select(conf, to_dev(dl_bad), cost, n, n, kept_o, budget,
                                        ws=bws))
    cap = n * (k + 1)
    maps = [torch.empty(cap, dtype=torch.int32, device="cuda") for _ in range(3)]
    cu_o = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    last = to_dev(np.arange(n, dtype=np.int32))
    sv.sv_pack_varlen(to_dev(kept.astype(np.int32)), last, toks_d, cu_o, *maps)
    kept_bad = kept.astype(np.int32).copy()
    kept_bad[2] = -1
    refused(lambda: sv.sv_pack_varlen(to_dev(kept_bad), last, toks_d, cu_o, *maps))

    # recorded under capture (the checks and the wait are skipped), then replayed
    for key, v in outs.items():
        v.fill_(-5)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        call(cu_d, toks_d)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(outs["tokens"].cpu().numpy(), ref["tokens"].cpu().numpy())


def test_end_to_end_path_on_device():
    """budget -> pack -> verify, each stage reading the previous stage's device output."""
    import adaptive_draft_verification_amd as sv
    w = workloads.make("b64_v128256")
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    o_b = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    toks = w.draft_tokens("stochastic")
    o_p = oracle.pack_varlen(o_b["kept"], w.last_token, toks, w.k_max)
    target = workloads.assemble_target(w, o_p["cu_rows"], o_b["kept"])
    draft = workloads.assemble_draft(w, o_b["kept"])
    dt = logits_dtype(w)
    b = sv.budget_select(to_dev(w.conf), to_dev(w.draft_len), to_dev(cost), w.t_base, w.n_bonus)
    p = sv.pack_varlen(b["kept"], to_dev(w.last_token), to_dev(toks))
    v = sv.verify(to_dev(target, dt), to_dev(draft, dt), to_dev(toks), p["cu_rows"],
                  sv.SV_STOCHASTIC, w.tau, w.seed, w.step)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(p["cu_rows"].cpu().numpy(), o_p["cu_rows"])
    g = {k: t.cpu().numpy() for k, t in v.items()}
    compare_verify(g, target, draft, toks, o_p["cu_rows"], w.k_max, w.vocab, "stochastic", w.tau,
                   w.seed, w.step)


def test_graph_replay_matches_eager():
    """The whole step captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit."""
    import adaptive_draft_verification_amd as sv
    w = workloads.make("b16_v32000")
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    o_b = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    toks = w.draft_tokens("stochastic")
    o_p = oracle.pack_varlen(o_b["kept"], w.last_token, toks, w.k_max)
    target = workloads.assemble_target(w, o_p["cu_rows"], o_b["kept"])
    draft = workloads.assemble_draft(w, o_b["kept"])
    dt = logits_dtype(w)
    n, k = w.n, w.k_max
    dev = torch.device("cuda")
    conf_d, dl_d, cost_d = to_dev(w.conf), to_dev(w.draft_len), to_dev(cost)
    last_d, toks_d = to_dev(w.last_token), to_dev(toks)
    tgt_d, drf_d = to_dev(target, dt), to_dev(draft, dt)
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(kept=torch.empty(n, **i32), budget=torch.empty(1, **i32),
               cu=torch.empty(n + 1, **i32), row_req=torch.empty(n * (k + 1), **i32),
               row_pos=torch.empty(n * (k + 1), **i32), packed=torch.empty(n * (k + 1), **i32),
               tokens=torch.empty(n, k + 1, **i32), accepted=torch.empty(n, **i32),
               err=torch.zeros(1, **i32))
    bws = torch.empty(max(1, sv.sv_budget_workspace_bytes(n, k)), dtype=torch.uint8, device=dev)
    vws = torch.zeros(sv.sv_verify_workspace_bytes(n, k), dtype=torch.uint8, device=dev)

    def step(s):
        sv.sv_budget_select(conf_d, dl_d, cost_d, w.t_base, w.n_bonus, out["kept"],
                            out["budget"], None, out["err"], ws=bws)
        sv.sv_pack_varlen(out["kept"], last_d, toks_d, out["cu"], out["row_req"],
                          out["row_pos"], out["packed"], out["err"])
        sv.sv_verify(tgt_d, drf_d, toks_d, out["cu"], sv.SV_STOCHASTIC, w.tau, w.seed, s,
                     out["tokens"], out["accepted"], vws, dev_error=out["err"], vocab=w.vocab)

    def snapshot():
        torch.cuda.synchronize()
        return {key: t.cpu().numpy().copy() for key, t in out.items()}

    step(5)
    want = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(5)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(5)
    for rep in range(4):
        step(6 + rep)  # eager work that changes every output in between
        other = snapshot()
        g.replay()
        got = snapshot()
        for key in want:
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"replay {rep}: {key}")
        assert not np.array_equal(other["tokens"], want["tokens"])
    assert int(want["err"][0]) == 0


def test_verify_reuses_an_uncleared_workspace():
    """Calls on one workspace that is never cleared (filled with garbage first):
    each equals a call on a fresh workspace."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(41)
    n, k, V = 24, 5, 70000
    target, draft, toks, cu = synthetic(rng, n, k, V)
    dt = torch.bfloat16
    t, d = to_dev(target, dt), to_dev(draft, dt)
    tk, cu_d = to_dev(toks), to_dev(cu)
    ws = torch.full((sv.sv_verify_workspace_bytes(n, k),), 0x5a, dtype=torch.uint8, device="cuda")
    for i, (mode, step) in enumerate([(sv.SV_STOCHASTIC, 3), (sv.SV_GREEDY, 0),
                                      (sv.SV_STOCHASTIC, 4), (sv.SV_STOCHASTIC, 4)]):
        got = sv.verify(t, d, tk, cu_d, mode, 0.9, 11, step, ws=ws)
        want = sv.verify(t, d, tk, cu_d, mode, 0.9, 11, step)
        torch.cuda.synchronize()
        for key in want:
            np.testing.assert_array_equal(got[key].cpu().numpy(), want[key].cpu().numpy(),
                                          err_msg=f"call {i}: {key}")


# ----------------------------------------- acceptance statistics, calibration

def random_outcomes(rng, n, k):
    kept = rng.integers(0, k + 1, n)
    cu = np.concatenate([[0], np.cumsum(kept + 1)]).astype(np.int32)
    L = np.array([rng.integers(0, b + 1) for b in kept], dtype=np.int32)
    L[rng.uniform(size=n) < 0.05] = -1          # faulted requests
    q = np.where(rng.uniform(size=(n, k)) < 0.05, 0.0,
                 rng.uniform(1e-4, 1.0, (n, k))).astype(np.float32)
    q[rng.uniform(size=(n, k)) < 0.01] = np.nan
    h = rng.uniform(0.0, 12.0, (n, k)).astype(np.float32)   # entropy, bits
    m = rng.uniform(1e-3, 1.0, (n, k)).astype(np.float32)   # largest probability
    for a in (h, m):  # not computed (-1) and NaN read as 0
        a[rng.uniform(size=(n, k)) < 0.02] = -1.0
        a[rng.uniform(size=(n, k)) < 0.01] = np.nan
    return L, cu, q, h, m


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (256, 7), (3000, 15), (100, 64), (5, 0)])
def test_accept_stats(n, k):
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(n * 7 + k)
    L, cu, _, _, _ = random_outcomes(rng, n, k)
    if n > 2:
        L[1] = (cu[2] - cu[1] - 1) + 1  # more accepted than kept: not a verify result
    att = torch.zeros(k, dtype=torch.int64, device="cuda")
    acc = torch.zeros(k, dtype=torch.int64, device="cuda")
    tot = torch.zeros(2, dtype=torch.int64, device="cuda")
    for _ in range(2):  # counters accumulate
        sv.sv_accept_stats(to_dev(L), to_dev(cu), att, acc, tot)
    torch.cuda.synchronize()
    o = oracle.accept_stats(L, cu, k)
    np.testing.assert_array_equal(att.cpu().numpy(), 2 * o["attempted"])
    np.testing.assert_array_equal(acc.cpu().numpy(), 2 * o["accepted_at"])
    assert tot.cpu().numpy().tolist() == [2 * o["requests"], 2 * o["emitted"]]


@pytest.mark.parametrize("features", [True, False])
@pytest.mark.parametrize("n,k,seed", [(1, 1, 0), (64, 7, 1), (2500, 7, 2), (300, 64, 3),
                                      (50, 3, 4)])
def test_calibrate_update_and_predict(n, k, seed, features):
    """fp32 on the device against the oracle's fp64, the count exact.  theta:
    relative 1e-5, absolute 1e-5 (a gradient component is a fixed-order fp32
    sum of up to ~2e4 terms |err * x| <= 12, divided by the count: its
    rounding stays below ~4e-6 per unit of lr).  conf: absolute 2e-6 (log2 of
    the fp32 probability to 1 ulp, about 1e-6 of the logit for |x_1| <= 16,
    times the sigmoid's slope <= 1/4, plus the fp32 sigmoid)."""
    import adaptive_draft_verification_amd as sv
    rng = np.random.default_rng(seed)
    L, cu, q, h, m = random_outcomes(rng, n, k)
    if not features:
        h = m = None
    dv = lambda a: None if a is None else to_dev(a)
    theta = rng.normal(0, 0.5, k + 3).astype(np.float32)
    th = to_dev(theta)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    sv.sv_calibrate_update(th, to_dev(q), to_dev(L), to_dev(cu), 0.5, cnt, q_entropy=dv(h),
                           q_max=dv(m))
    torch.cuda.synchronize()
    want, count = oracle.calibrate_update(theta.astype(np.float64), q, L, cu, k, 0.5, h, m)
    assert int(cnt.cpu()[0]) == count
    np.testing.assert_allclose(th.cpu().numpy(), want, rtol=1e-5, atol=1e-5)
    conf = torch.empty(n, k, dtype=torch.float32, device="cuda")
    sv.sv_calibrate_predict(th, to_dev(q), conf, q_entropy=dv(h), q_max=dv(m))
    torch.cuda.synchronize()
    np.testing.assert_allclose(
        conf.cpu().numpy(),
        oracle.calibrate_predict(th.cpu().numpy().astype(np.float64), q, k, h, m),
        rtol=2e-6, atol=2e-6)


def test_calibration_from_a_verify_step():
    """budget -> pack -> verify on the device, then the step's statistics and one
    calibration step from the verify outputs, each against the oracle fed the
    same outputs."""
    import adaptive_draft_verification_amd as sv
    w = workloads.make("b64_v128256")
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    o_b = oracle.budget_select(w.conf, w.draft_len, w.k_max, cost, w.t_base, w.n_bonus)
    toks = w.draft_tokens("stochastic")
    o_p = oracle.pack_varlen(o_b["kept"], w.last_token, toks, w.k_max)
    target = workloads.assemble_target(w, o_p["cu_rows"], o_b["kept"])
    draft = workloads.assemble_draft(w, o_b["kept"])
    dt = logits_dtype(w)
    b = sv.budget_select(to_dev(w.conf), to_dev(w.draft_len), to_dev(cost), w.t_base, w.n_bonus)
    p = sv.pack_varlen(b["kept"], to_dev(w.last_token), to_dev(toks))
    v = sv.verify(to_dev(target, dt), to_dev(draft, dt), to_dev(toks), p["cu_rows"],
                  sv.SV_STOCHASTIC, w.tau, w.seed, w.step, features=True)
    k = w.k_max
    att = torch.zeros(k, dtype=torch.int64, device="cuda")
    acc = torch.zeros(k, dtype=torch.int64, device="cuda")
    tot = torch.zeros(2, dtype=torch.int64, device="cuda")
    sv.sv_accept_stats(v["accepted"], p["cu_rows"], att, acc, tot)
    theta = torch.zeros(k + 3, dtype=torch.float32, device="cuda")
    sv.sv_calibrate_update(theta, v["q_draft"], v["accepted"], p["cu_rows"], 1.0,
                           q_entropy=v["q_entropy"], q_max=v["q_max"])
    torch.cuda.synchronize()
    L = v["accepted"].cpu().numpy()
    cu = p["cu_rows"].cpu().numpy()
    q = v["q_draft"].cpu().numpy()
    h, m = v["q_entropy"].cpu().numpy(), v["q_max"].cpu().numpy()
    o = oracle.accept_stats(L, cu, k)
    np.testing.assert_array_equal(att.cpu().numpy(), o["attempted"])
    np.testing.assert_array_equal(acc.cpu().numpy(), o["accepted_at"])
    assert tot.cpu().numpy().tolist() == [o["requests"], o["emitted"]] and o["requests"] == w.n
    want, _ = oracle.calibrate_update(np.zeros(k + 3), q, L, cu, k, 1.0, h, m)
    np.testing.assert_allclose(theta.cpu().numpy(), want, rtol=1e-5, atol=1e-5)
    # the features themselves: the oracle's, at the kept positions
    for r in range(0, w.n, 7):
        for j in range(int(o_b["kept"][r])):
            eh, em = oracle.draft_features(draft[r * k + j, : w.vocab], w.tau)
            assert abs(h[r, j] - eh) <= H_ATOL + H_RTOL * eh and abs(m[r, j] - em) <= P_RTOL * em
