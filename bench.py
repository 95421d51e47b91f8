"""Benchmark of the verify step on one MI355X.

A step is one pass of the whole path on one batch: adaptive budget selection
(sv_budget_select), varlen packing (sv_pack_varlen) and full-vocabulary
verification (sv_verify: pass 1 row statistics, pass 2 decisions and draws),
each stage reading the previous stage's device output.  The default workload
is 256 requests with 7 drafts each over a 129280-token vocabulary, bf16
logits, confidences X^j with X ~ Beta(8, 2), and a cost table padded to
multiples of 16 tokens (workloads.make("b256_v129280")); the budget decides
how many rows each request verifies.

Inputs are generated once on the host and copied to HBM before timing; two
replicas of the logit buffers alternate between steps so that reads come from
HBM rather than the 256 MB Infinity Cache.  HIP events on the launch stream
time every stage; `value` is target rows verified per second of whole-step
time.  A second leg verifies every draft (full K: 2048 target + 1792 draft
rows) for the bandwidth figure at the largest size.  The CPU oracle runs one
step of the same workload on the host for the cpu_baseline figure.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = ("verify rows/sec (K+1 rows/req × vocab) + achieved HBM GB/s; "
          "budget-select µs/step")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="b256_v129280")
    ap.add_argument("--mode", choices=["stochastic", "greedy"], default="stochastic")
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--full-k-iters", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="lower bound on the oracle's timed host work")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); the verify step shards by request with no "
              f"exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import torch

    import adaptive_draft_verification_amd as sv
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = workloads.make(args.workload)
    mode = sv.SV_GREEDY if args.mode == "greedy" else sv.SV_STOCHASTIC
    ldt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esize = 2 if w.dtype == "bf16" else 4
    n, K, V = w.n, w.k_max, w.vocab

    t0 = time.time()
    # full logits: target row (r, j) at r*(K+1) + j, draft row (r, j) at r*K + j
    tgt_full = np.full((n * (K + 1), V), np.nan, dtype=np.float32)
    drf_full = np.full((n * K, V), np.nan, dtype=np.float32)
    tok_key = "tok_greedy" if args.mode == "greedy" else "tok_stochastic"
    toks_np = np.full((n, K), -1, dtype=np.int32)
    for r in range(n):
        rq = w.request(r)
        Kr = int(w.draft_len[r])
        tgt_full[r * (K + 1): r * (K + 1) + Kr + 1] = rq["target"]
        drf_full[r * K: r * K + Kr] = rq["draft"]
        toks_np[r] = rq[tok_key]
        w.drop_cache()
    print(f"[bench] generated {args.workload} in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    def d(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.to(dtype) if dtype is not None else t).to(dev)

    cost = sv.sv_cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
    conf_d, dl_d, cost_d = d(w.conf), d(w.draft_len), d(cost)
    last_d, toks_d = d(w.last_token), d(toks_np)
    tgt_full_d = d(tgt_full, ldt)
    drf_full_d = d(drf_full, ldt)

    # outputs and workspace, allocated once
    kept = torch.empty(n, dtype=torch.int32, device=dev)
    budget = torch.empty(1, dtype=torch.int32, device=dev)
    survival = torch.empty(n, K, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    cap = n * (K + 1)
    cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
    row_req = torch.empty(cap, dtype=torch.int32, device=dev)
    row_pos = torch.empty(cap, dtype=torch.int32, device=dev)
    packed = torch.empty(cap, dtype=torch.int32, device=dev)
    ws = torch.empty(sv.sv_verify_workspace_bytes(n, K), dtype=torch.uint8, device=dev)
    tok_out = torch.empty(n, K + 1, dtype=torch.int32, device=dev)
    acc_out = torch.empty(n, dtype=torch.int32, device=dev)
    p_out = torch.empty(n, K, dtype=torch.float32, device=dev)
    q_out = torch.empty(n, K, dtype=torch.float32, device=dev)
    res_out = torch.empty(n, dtype=torch.float32, device=dev)

    # set-up pass: the budget's packing decides which target rows the (stand-in)
    # target forward would produce; gather them once into packed buffers
    sv.sv_budget_select(conf_d, dl_d, cost_d, w.t_base, w.n_bonus, kept, budget, survival, err)
    sv.sv_pack_varlen(kept, last_d, toks_d, cu, row_req, row_pos, packed, err)
    torch.cuda.synchronize()
    kept_h = kept.cpu().numpy()
    cu_h = cu.cpu().numpy()
    B = int(budget.item())
    rows_t = int(cu_h[-1])
    rows_d = int(kept_h.sum())
    idx = np.concatenate([r * (K + 1) + np.arange(int(kept_h[r]) + 1) for r in range(n)])
    idx_d = d(idx.astype(np.int64))
    replicas = []
    for i in range(args.replicas):
        tp = torch.full((cap, V), float("nan"), dtype=ldt, device=dev)
        tp[:rows_t] = tgt_full_d.index_select(0, idx_d)
        dr = drf_full_d if i == 0 else drf_full_d.clone()
        replicas.append((tp, dr))
    torch.cuda.synchronize()

    def step(i, events=None):
        tp, dr = replicas[i % len(replicas)]
        if events is not None:
            events[0].record(stream)
        sv.sv_budget_select(conf_d, dl_d, cost_d, w.t_base, w.n_bonus, kept, budget, survival,
                            err)
        if events is not None:
            events[1].record(stream)
        sv.sv_pack_varlen(kept, last_d, toks_d, cu, row_req, row_pos, packed, err)
        if events is not None:
            events[2].record(stream)
        sv.sv_verify_stages(tp, dr, toks_d, cu, mode, w.tau, w.seed, i, tok_out, acc_out, ws, 1,
                            p_out, q_out, res_out, err, vocab=V)
        if events is not None:
            events[3].record(stream)
        sv.sv_verify_stages(tp, dr, toks_d, cu, mode, w.tau, w.seed, i, tok_out, acc_out, ws, 2,
                            p_out, q_out, res_out, err, vocab=V)
        if events is not None:
            events[4].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage_ms = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(4)]
                         for i in range(args.steps)])
    gpu_step_ms = np.array([ev[i][0].elapsed_time(ev[i][4]) for i in range(args.steps)])
    if int(err.item()) != 0:
        raise RuntimeError(f"device error bits {int(err.item())} during the benchmark")
    # pass-2 bytes depend on the draws (a rejection re-reads two rows, an
    # all-accepted request one): take them from one more step
    step(args.steps)
    torch.cuda.synchronize()
    acc_h = acc_out.cpu().numpy()
    n_rejected = int(((acc_h >= 0) & (acc_h < kept_h)).sum())

    ms_per_step = wall * 1e3 / args.steps
    pass1_ms = float(np.mean(stage_ms[:, 2]))
    pass1_bytes = (rows_t + (rows_d if mode == sv.SV_STOCHASTIC else 0)) * V * esize
    pass2_bytes = (n_rejected * 2 + (n - n_rejected)) * V * esize if mode == sv.SV_STOCHASTIC \
        else 0
    achieved = pass1_bytes / (pass1_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- full K leg
    full = None
    if args.full_k_iters > 0:
        cu_full = torch.empty(n + 1, dtype=torch.int32, device=dev)
        sv.sv_pack_varlen(dl_d, last_d, toks_d, cu_full, row_req, row_pos, packed, err)
        full_reps = [(tgt_full_d, drf_full_d)]
        if args.replicas > 1:
            full_reps.append((tgt_full_d.clone(), replicas[1][1]))
        rows_tf = int(cu_full[-1].item())
        rows_df = int(w.draft_len.sum())
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.full_k_iters)]
        for i in range(3):
            tp, dr = full_reps[i % len(full_reps)]
            sv.sv_verify(tp, dr, toks_d, cu_full, mode, w.tau, w.seed, i, tok_out, acc_out, ws,
                         p_out, q_out, res_out, err, vocab=V)
        torch.cuda.synchronize()
        for i in range(args.full_k_iters):
            tp, dr = full_reps[i % len(full_reps)]
            fev[i][0].record(stream)
            sv.sv_verify_stages(tp, dr, toks_d, cu_full, mode, w.tau, w.seed, i, tok_out,
                                acc_out, ws, 1, p_out, q_out, res_out, err, vocab=V)
            fev[i][1].record(stream)
            sv.sv_verify_stages(tp, dr, toks_d, cu_full, mode, w.tau, w.seed, i, tok_out,
                                acc_out, ws, 2, p_out, q_out, res_out, err, vocab=V)
            fev[i][2].record(stream)
        torch.cuda.synchronize()
        f1 = float(np.mean([fev[i][0].elapsed_time(fev[i][1]) for i in range(args.full_k_iters)]))
        f2 = float(np.mean([fev[i][1].elapsed_time(fev[i][2]) for i in range(args.full_k_iters)]))
        fbytes = (rows_tf + (rows_df if mode == sv.SV_STOCHASTIC else 0)) * V * esize
        acc_f = acc_out.cpu().numpy()
        nrej_f = int(((acc_f >= 0) & (acc_f < w.draft_len)).sum())
        fbytes2 = (nrej_f * 2 + (n - nrej_f)) * V * esize if mode == sv.SV_STOCHASTIC else 0
        full = {
            "target_rows": rows_tf, "draft_rows": rows_df if mode == sv.SV_STOCHASTIC else 0,
            "pass1_us": round(f1 * 1e3, 2), "pass2_us": round(f2 * 1e3, 2),
            "pass1_gbps": round(fbytes / (f1 * 1e-3) / 1e9, 1),
            "pass1_frac": round(fbytes / (f1 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "verify_gbps": round((fbytes + fbytes2) / ((f1 + f2) * 1e-3) / 1e9, 1),
            "verify_frac": round((fbytes + fbytes2) / ((f1 + f2) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "verify_rows_per_s": round(rows_tf / ((f1 + f2) * 1e-3), 1),
            "iters": args.full_k_iters,
        }
        if int(err.item()) != 0:
            raise RuntimeError(f"device error bits {int(err.item())} in the full-K leg")

    # ------------------------------------------------------------ CPU oracle leg
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tp_h = tgt_full[idx]
        omode = oracle.GREEDY if mode == sv.SV_GREEDY else oracle.STOCHASTIC
        steps_cpu, rows_cpu = 0, 0
        t_c = time.perf_counter()
        while steps_cpu == 0 or time.perf_counter() - t_c < args.cpu_seconds:
            cost_o = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
            ob = oracle.budget_select(w.conf, w.draft_len, K, cost_o, w.t_base, w.n_bonus)
            op = oracle.pack_varlen(ob["kept"], w.last_token, toks_np, K)
            oracle.verify(tp_h, drf_full if mode == sv.SV_STOCHASTIC else None, toks_np,
                          op["cu_rows"], K, V, omode, w.tau, w.seed, steps_cpu)
            steps_cpu += 1
            rows_cpu += int(op["cu_rows"][-1])
        t_cpu = time.perf_counter() - t_c
        cpu = {"value": round(rows_cpu / t_cpu, 2), "unit": "rows/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{steps_cpu} whole steps of {args.workload} (budget, pack, {args.mode} "
                         f"verify of {rows_t} target rows each, Philox step varied) with numpy "
                         f"fp64 on one host thread, {t_cpu:.1f} s"}

    out = {
        "metric": METRIC,
        "value": round(rows_t / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "n_req": n, "k": K, "vocab": V,
            "logits": w.dtype, "mode": args.mode, "temperature": w.tau,
            "budget": B, "target_rows": rows_t, "draft_rows": rows_d,
            "cost_granule": w.granule,
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "rowstats_kernel (verify pass 1)",
                     "bytes_per_launch": pass1_bytes},
        "budget_select_us": round(float(np.mean(stage_ms[:, 0])) * 1e3, 2),
        "pack_us": round(float(np.mean(stage_ms[:, 1])) * 1e3, 2),
        "verify_pass1_us": round(pass1_ms * 1e3, 2),
        "verify_pass2_us": round(float(np.mean(stage_ms[:, 3])) * 1e3, 2),
        "gpu_step_us": round(float(np.mean(gpu_step_ms)) * 1e3, 2),
        "step_hbm_gbps": round((pass1_bytes + pass2_bytes) / (ms_per_step * 1e-3) / 1e9, 1),
        "full_k": full,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
