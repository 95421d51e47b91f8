"""Benchmark of the verify step on one MI355X.

A step is one pass of the whole path on one batch: adaptive budget selection
and varlen packing (sv_budget_select_pack: the two in one launch fewer;
--separate-pack calls sv_budget_select and sv_pack_varlen) and full-vocabulary
verification (sv_verify: row statistics, then one workgroup per request that
decides and draws), each stage reading the previous stage's device output.
The default workload is 256 requests with 7 drafts each over a 129280-token
vocabulary, bf16 logits, confidences X^j with X ~ Beta(8, 2), and a cost
table padded to multiples of 16 tokens (workloads.make("b256_v129280")); the
budget decides how many rows each request verifies.

Inputs are generated once on the host and copied to HBM before timing; four
replicas of the logit buffers (about 1 GB each) rotate between steps so that
reads come from HBM rather than the 256 MB Infinity Cache: with two, the rows
a draw re-read two steps earlier could still be cached when pass 1 streams
that replica again.  The headline times K steps
launched back to back (--graph replays them from HIP graphs instead, one per
replica and Philox step, in turn); `value` is target rows verified per second
of that wall time.  A separate loop with HIP events on the launch stream times
every stage; the roofline is pass 1's algorithmic bytes (every kept row once)
over its mean launch time (K launches back to back between two events), with
the HBM bytes the byte counters measured for it
(profiles/, while the kernel's sources are unchanged); pass 2's bytes (the
rows each draw reads again) are reported beside it.  A second leg verifies
every draft (full K: 2048 target + 1792 draft rows) for the bandwidth figure
at the largest size.  Two smaller legs time pass 1 with the draft-row
features (entropy, largest probability) accumulated as well, and the one-K-
per-batch selection (sv_uniform_k_select), the allocation of a budget
sized one step ahead (sv_budget_allocate), and the acceptance counters and
the logistic calibration's update and prediction fed by one verify step
(sv_accept_stats, sv_calibrate_update, sv_calibrate_predict).  Before the GPU is touched, the CPU
oracle runs whole steps of the same workload on the host for the cpu_baseline
figure: half the time on one thread, half with each step's requests spread
over a pool of worker processes (the reported value; the one-thread rate is in
its sample text).

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
SMALL_CALL_ITERS = 1000  # graph-replayed calls per figure for the microsecond entry points
METRIC = ("verify rows/sec (K+1 rows/req × vocab) + achieved HBM GB/s; "
          "budget-select µs/step")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="b256_v129280")
    ap.add_argument("--mode", choices=["stochastic", "greedy"], default="stochastic")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--full-k-iters", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="lower bound on the oracle's timed host work")
    ap.add_argument("--graph", dest="graph", action="store_true", default=False,
                    help="time steps replayed from HIP graphs (slower than eager launches "
                         "on ROCm 7.2: ~130 vs ~122 us per step)")
    ap.add_argument("--eager", dest="graph", action="store_false",
                    help="time eagerly launched steps (default)")
    ap.add_argument("--graphs", type=int, default=4,
                    help="graphs captured (one per replica and Philox step), replayed in turn")
    ap.add_argument("--separate-pack", action="store_true",
                    help="budget and pack as two calls (sv_budget_select, sv_pack_varlen) "
                         "instead of sv_budget_select_pack")
    ap.add_argument("--all-drafts", action="store_true",
                    help="the timed step verifies every draft (full K) of the workload; budget "
                         "and pack still run in the step, but verify reads the full-K packing "
                         "(for profiling the largest size on its own)")
    ap.add_argument("--legs", default="greedy,mix",
                    help="secondary legs after the headline: greedy (same workload, greedy "
                         "mode), mix (256 requests, K_r up to 15, V = 256000, fp32); 'none'")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only copy a device buffer of this many MiB three times and exit: "
                         "a plain copy of known size, to scale HBM byte counters by")
    return ap.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "verify_pass1_b256_v129280_hbm_bytes.md")


def measured_traffic(workload, mode):
    """Pass-1 HBM bytes per launch from the committed rocprofv3 byte-counter
    summary, or None unless it covers this workload and mode and the kernel's
    sources still hash as they did when the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    wl = re.search(r"^workload: (\S+) (\S+)$", text, re.M)
    tb = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    hs = re.search(r"^sources_sha256: ([0-9a-f]{64})$", text, re.M)
    srcs = re.search(r"^sources: (.+)$", text, re.M)
    if not (wl and tb and hs and srcs) or wl.groups() != (workload, mode):
        return None
    h = hashlib.sha256()
    for f in srcs.group(1).split():
        try:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        except OSError:
            return None
    return int(tb.group(1)) if h.hexdigest() == hs.group(1) else None


def copy_calibration(mib):
    """Three device-to-device copies of `mib` MiB (read mib, write mib each)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


# Inputs the forked oracle workers read (set before the pool forks; the
# workers only read them, so the pages are shared, not copied).
_CPU = {}


def _oracle_requests(job):
    """Oracle verify of requests [r0, r1) of one step (a pool worker's share)."""
    import oracle
    r0, r1, step = job
    c = _CPU
    K, V = c["K"], c["V"]
    rows = 0
    for r in range(r0, r1):
        b = int(c["kept"][r])
        trows = [c["tgt"][r * (K + 1) + j, :V] for j in range(b + 1)]
        drows = [] if c["greedy"] else [c["drf"][r * K + j, :V] for j in range(b)]
        oracle.verify_request(r, trows, drows, c["toks"][r], b, V, c["omode"], c["tau"],
                              c["seed"], step)
        rows += b + 1
    return rows


def cpu_baseline(args, w, tgt_full, drf_full, toks_np):
    """The oracle on the host, before anything touches the GPU: whole steps
    (budget, pack, verify) on one thread, then with the requests of each step
    spread over a pool of worker processes (budget and pack stay in the
    parent).  Returns the cpu_baseline object (the pool's figure)."""
    import multiprocessing as mp

    import oracle
    K, V, n = w.k_max, w.vocab, w.n
    greedy = args.mode == "greedy"
    omode = oracle.GREEDY if greedy else oracle.STOCHASTIC
    cost = oracle.cost_table_prepare(w.raw_cost, w.granule, w.cost_len)

    def budget_and_pack():
        ob = oracle.budget_select(w.conf, w.draft_len, K, cost, w.t_base, w.n_bonus)
        op = oracle.pack_varlen(ob["kept"], w.last_token, toks_np, K)
        return ob["kept"], op["cu_rows"]

    kept, cu = budget_and_pack()
    # the packed target rows a varlen forward would write for this budget
    idx = np.concatenate([r * (K + 1) + np.arange(int(kept[r]) + 1) for r in range(n)])
    tp_h = tgt_full[idx]
    half = args.cpu_seconds / 2

    steps1, rows1 = 0, 0
    t_c = time.perf_counter()
    while steps1 == 0 or time.perf_counter() - t_c < half:
        kept, cu = budget_and_pack()
        oracle.verify(tp_h, None if greedy else drf_full, toks_np, cu, K, V, omode, w.tau,
                      w.seed, steps1)
        steps1 += 1
        rows1 += int(cu[-1])
    t1 = time.perf_counter() - t_c

    # one worker process per CPU this process may run on, at most 16: the host
    # CPUs allotted to a one-GPU job (more processes would compete for them)
    host_cpus = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cpus))
    _CPU.update(K=K, V=V, kept=kept, tgt=tgt_full, drf=drf_full, toks=toks_np, greedy=greedy,
                omode=omode, tau=w.tau, seed=w.seed)
    chunks = min(n, 4 * workers)
    bounds = [n * i // chunks for i in range(chunks + 1)]
    steps2, rows2 = 0, 0
    with mp.get_context("fork").Pool(workers) as pool:
        t_c = time.perf_counter()
        while steps2 == 0 or time.perf_counter() - t_c < half:
            kept_s, cu = budget_and_pack()
            jobs = [(bounds[i], bounds[i + 1], steps2) for i in range(chunks)]
            rows2 += sum(pool.map(_oracle_requests, jobs))
            steps2 += 1
        t2 = time.perf_counter() - t_c
    _CPU.clear()
    rows_step = int(cu[-1])
    return {"value": round(rows2 / t2, 2), "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": f"{steps2} whole steps of {args.workload} (budget and pack in the parent, "
                      f"{args.mode} verify of {rows_step} target rows each spread over {workers} "
                      f"worker processes, Philox step varied) with numpy fp64, {t2:.1f} s; on one "
                      f"thread {steps1} steps in {t1:.1f} s = {rows1 / t1:.2f} rows/s",
            "single_thread_value": round(rows1 / t1, 2),
            "host_cpus": host_cpus, "host_cpus_total": os.cpu_count(),
            "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's guess."""
    import platform
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Leg:
    """Device state for timing one workload in one mode: inputs, outputs, the
    workspaces, and `replicas` copies of the packed target rows and the draft
    rows (reads then come from HBM, not the 256 MB Infinity Cache).  `share`
    reuses another leg's logit replicas and budget (same workload, other mode)."""

    def __init__(self, sv, torch, w, mode_name, tgt_full_d, drf_full_d, toks_np, args,
                 share=None):
        self.sv, self.torch, self.w, self.args = sv, torch, w, args
        self.mode = sv.SV_GREEDY if mode_name == "greedy" else sv.SV_STOCHASTIC
        self.mode_name = mode_name
        dev = self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        n, K, V = w.n, w.k_max, w.vocab
        self.esize = 2 if w.dtype == "bf16" else 4

        def d(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.to(dtype) if dtype is not None else t).to(dev)

        self.d = d
        self.cost = sv.sv_cost_table_prepare(w.raw_cost, w.granule, w.cost_len)
        self.conf_d, self.dl_d, self.cost_d = d(w.conf), d(w.draft_len), d(self.cost)
        self.last_d, self.toks_d = d(w.last_token), d(toks_np)
        self.tgt_full_d, self.drf_full_d = tgt_full_d, drf_full_d
        e = lambda *shape, dt=torch.int32: torch.empty(*shape, dtype=dt, device=dev)
        self.kept, self.budget, self.err = e(n), e(1), torch.zeros(1, dtype=torch.int32, device=dev)
        self.survival = e(n, K, dt=torch.float32)
        self.cap = cap = n * (K + 1)
        self.cu, self.row_req, self.row_pos, self.packed = e(n + 1), e(cap), e(cap), e(cap)
        self.verify_cu = self.cu  # the packing verify reads (the step's own by default)
        self.ws = torch.zeros(sv.sv_verify_workspace_bytes(n, K), dtype=torch.uint8, device=dev)
        self.bws = torch.empty(max(1, sv.sv_budget_workspace_bytes(n, K)), dtype=torch.uint8,
                               device=dev)
        self.tok_out, self.acc_out = e(n, K + 1), e(n)
        self.p_out, self.q_out = e(n, K, dt=torch.float32), e(n, K, dt=torch.float32)
        self.res_out = e(n, dt=torch.float32)

        # set-up pass: the budget's packing decides which target rows the (stand-in)
        # target forward would produce; gather them once into packed buffers
        sv.sv_budget_select(self.conf_d, self.dl_d, self.cost_d, w.t_base, w.n_bonus, self.kept,
                            self.budget, self.survival, self.err, ws=self.bws)
        sv.sv_pack_varlen(self.kept, self.last_d, self.toks_d, self.cu, self.row_req,
                          self.row_pos, self.packed, self.err)
        torch.cuda.synchronize()
        self.kept_h = self.kept.cpu().numpy()
        self.B = int(self.budget.item())
        self.rows_t = int(self.cu[-1].item())
        self.rows_d = int(self.kept_h.sum())
        if share is not None:
            self.replicas = share.replicas
        else:
            idx = np.concatenate([r * (K + 1) + np.arange(int(self.kept_h[r]) + 1)
                                  for r in range(n)])
            idx_d = d(idx.astype(np.int64))
            self.replicas = []
            for i in range(args.replicas):
                tp = torch.full((cap, V), float("nan"), dtype=tgt_full_d.dtype, device=dev)
                tp[: self.rows_t] = tgt_full_d.index_select(0, idx_d)
                dr = drf_full_d if i == 0 else drf_full_d.clone()
                self.replicas.append((tp, dr))
        torch.cuda.synchronize()

    def step(self, i, events=None, reps=None, cu_rows=None, kept_in=None):
        """One step; events (5) bracket budget, pack, verify pass 1, verify pass 2."""
        sv, w = self.sv, self.w
        tp, dr = (reps or self.replicas)[i % len(reps or self.replicas)]
        cu_i = self.verify_cu if cu_rows is None else cu_rows

        def mark(k):
            if events is not None:
                events[k].record(self.stream)

        mark(0)
        if kept_in is None and self.args.separate_pack:
            sv.sv_budget_select(self.conf_d, self.dl_d, self.cost_d, w.t_base, w.n_bonus,
                                self.kept, self.budget, self.survival, self.err, ws=self.bws)
            mark(1)
            sv.sv_pack_varlen(self.kept, self.last_d, self.toks_d, self.cu, self.row_req,
                              self.row_pos, self.packed, self.err)
        elif kept_in is None:  # budget and pack in one launch fewer
            sv.sv_budget_select_pack(self.conf_d, self.dl_d, self.cost_d, w.t_base, w.n_bonus,
                                     self.last_d, self.toks_d, self.kept, self.budget, self.cu,
                                     self.row_req, self.row_pos, self.packed, self.survival,
                                     self.err, ws=self.bws)
            mark(1)
        else:
            mark(1)
        mark(2)
        for stage in (1, 2):
            sv.sv_verify_stages(tp, dr, self.toks_d, cu_i, self.mode, w.tau, w.seed, i,
                                self.tok_out, self.acc_out, self.ws, stage, self.p_out,
                                self.q_out, self.res_out, self.err, vocab=w.vocab)
            mark(2 + stage)

    def pass2_ids(self, steps, kept_h_, **kw):
        """Logits the draws must re-read in each of `steps` (deterministic: same step
        index, same draws): both rows whole for a rejected request (the residual's
        total needs every id), and for a request that accepted every draft the bonus
        row's ids up to the drawn one (its total comes from pass 1, so the draw's
        sweep stops once it has passed the drawn id)."""
        if self.mode == self.sv.SV_GREEDY:
            return np.zeros(len(steps))
        out = []
        V = self.w.vocab
        kept = np.asarray(kept_h_)
        for i in steps:
            self.step(i, **kw)
            acc = self.acc_out.cpu().numpy()
            tok = self.tok_out.cpu().numpy()
            rej = (acc >= 0) & (acc < kept)
            bonus = (acc >= 0) & (acc == kept)
            drawn = tok[np.arange(len(acc)), np.clip(acc, 0, None)]
            out.append(2 * V * int(rej.sum()) + int((drawn[bonus] + 1).sum()))
        return np.array(out, dtype=np.float64)

    def timed(self, iters, **kw):
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(iters)]
        torch.cuda.synchronize()
        t0_ = time.perf_counter()
        for i in range(iters):
            self.step(i, ev[i], **kw)
        torch.cuda.synchronize()
        wall_ = time.perf_counter() - t0_
        ms = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(4)]
                       for i in range(iters)])
        if int(self.err.item()) != 0:
            raise RuntimeError(f"device error bits {int(self.err.item())} during the benchmark")
        return wall_, ms

    def pass1_launch_ms(self, iters, reps=None, cu_rows=None, features=False):
        """Mean duration of the roofline kernel: `iters` pass-1 launches back to
        back (replicas in turn) between two events on the launch stream.
        features: the launch that also accumulates the draft-row features."""
        sv, torch, w = self.sv, self.torch, self.w
        reps = reps or self.replicas
        cu_i = self.verify_cu if cu_rows is None else cu_rows
        fkw = {}
        if features:
            fkw = dict(out_q_entropy=torch.empty(w.n, w.k_max, dtype=torch.float32,
                                                 device=self.dev),
                       out_q_max=torch.empty(w.n, w.k_max, dtype=torch.float32,
                                             device=self.dev))
        for i in range(2):
            tp_, dr_ = reps[i % len(reps)]
            sv.sv_verify_stages(tp_, dr_, self.toks_d, cu_i, self.mode, w.tau, w.seed, i,
                                self.tok_out, self.acc_out, self.ws, 1, self.p_out, self.q_out,
                                self.res_out, self.err, vocab=w.vocab, **fkw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(iters):
            tp_, dr_ = reps[i % len(reps)]
            sv.sv_verify_stages(tp_, dr_, self.toks_d, cu_i, self.mode, w.tau, w.seed, i,
                                self.tok_out, self.acc_out, self.ws, 1, self.p_out, self.q_out,
                                self.res_out, self.err, vocab=w.vocab, **fkw)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def verify_launch_ms(self, iters):
        """Mean duration of the whole verify call (both passes, no event between
        them): `iters` calls back to back (replicas in turn) between two events on
        the launch stream, the same draws as the step's."""
        sv, torch, w = self.sv, self.torch, self.w
        reps = self.replicas

        def call(i):
            tp_, dr_ = reps[i % len(reps)]
            sv.sv_verify_stages(tp_, dr_, self.toks_d, self.verify_cu, self.mode, w.tau, w.seed,
                                i, self.tok_out, self.acc_out, self.ws, 3, self.p_out,
                                self.q_out, self.res_out, self.err, vocab=w.vocab)
        for i in range(2):
            call(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(iters):
            call(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def full_k_inputs(self):
        """Every draft kept: request r's rows 0..K_r packed at cu_full[r] (the layout a
        varlen target forward writes), gathered from the per-request stride K+1."""
        sv, torch, w = self.sv, self.torch, self.w
        n, K = w.n, w.k_max
        cu_full = torch.empty(n + 1, dtype=torch.int32, device=self.dev)
        sv.sv_pack_varlen(self.dl_d, self.last_d, self.toks_d, cu_full, self.row_req,
                          self.row_pos, self.packed, self.err)
        full_idx = np.concatenate([r * (K + 1) + np.arange(int(w.draft_len[r]) + 1)
                                   for r in range(n)])
        tgt_packed = self.tgt_full_d.index_select(0, self.d(full_idx.astype(np.int64)))
        reps = [(tgt_packed if i == 0 else tgt_packed.clone(), self.replicas[i][1])
                for i in range(len(self.replicas))]
        rows_tf = int(cu_full[-1].item())
        rows_df = int(w.draft_len.sum()) if self.mode == sv.SV_STOCHASTIC else 0
        return reps, cu_full, rows_tf, rows_df

    def pass1_bytes(self, rows_t, rows_d):
        rd = rows_d if self.mode == self.sv.SV_STOCHASTIC else 0
        return (rows_t + rd) * self.w.vocab * self.esize

    def leg_figures(self, steps, full_k_iters):
        """The figures reported for a secondary leg: eager steps back to back, the
        staged loop, pass 1 back to back (adaptive and full K), pass 2's bytes."""
        run = lambda i: self.step(i)
        for i in range(3):
            self.step(i)
        wall = timed_plain(self.torch, steps, run)
        for i in range(2):
            self.step(i)
        _, stage_ms = self.timed(steps)
        p2_ids = self.pass2_ids(range(steps), self.kept_h)
        p1_ms = self.pass1_launch_ms(steps)
        p1_bytes = self.pass1_bytes(self.rows_t, self.rows_d)
        p2_bytes = float(np.mean(p2_ids)) * self.esize
        p2_ms = float(np.mean(stage_ms[:, 3]))
        out = {
            "workload": self.w.name, "mode": self.mode_name, "logits": self.w.dtype,
            "temperature": self.w.tau, "budget": self.B, "target_rows": self.rows_t,
            "draft_rows": self.rows_d if self.mode == self.sv.SV_STOCHASTIC else 0,
            "step_us": round(wall * 1e6 / steps, 2),
            "rows_per_s": round(self.rows_t / (wall / steps), 1),
            "budget_pack_us": round(float(np.mean(stage_ms[:, 0] + stage_ms[:, 1])) * 1e3, 2),
            "pass1_us": round(p1_ms * 1e3, 2), "pass1_bytes": int(p1_bytes),
            "pass1_gbps": round(p1_bytes / (p1_ms * 1e-3) / 1e9, 1),
            "pass1_frac": round(p1_bytes / (p1_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "pass2_us": round(p2_ms * 1e3, 2), "pass2_bytes": int(p2_bytes),
        }
        if p2_bytes > 0:
            out["pass2_gbps"] = round(p2_bytes / (p2_ms * 1e-3) / 1e9, 1)
            out["pass2_frac"] = round(p2_bytes / (p2_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if full_k_iters > 0:
            reps, cu_full, rows_tf, rows_df = self.full_k_inputs()
            f_ms = self.pass1_launch_ms(full_k_iters, reps=reps, cu_rows=cu_full)
            f_bytes = self.pass1_bytes(rows_tf, rows_df)
            out["full_k"] = {"target_rows": rows_tf, "draft_rows": rows_df,
                             "pass1_us": round(f_ms * 1e3, 2), "pass1_bytes": int(f_bytes),
                             "pass1_gbps": round(f_bytes / (f_ms * 1e-3) / 1e9, 1),
                             "pass1_frac": round(f_bytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                                 4)}
        return out


def timed_plain(torch, iters, fn):
    """Wall time of `iters` calls of fn with nothing else on the stream."""
    torch.cuda.synchronize()
    t0_ = time.perf_counter()
    for i in range(iters):
        fn(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0_


def step_percentiles(torch, stream, iters, fn):
    """p10, median and p90 of one step's time (us): an event at every step
    boundary of `iters` steps launched back to back on `stream`."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    for i in range(iters):
        ev[i].record(stream)
        fn(i)
    ev[iters].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]) * 1e3
    return [round(float(np.percentile(us, q)), 2) for q in (10, 50, 90)]


def graph_us(torch, fn, iters):
    """GPU time per call of a small entry point: `iters` calls captured in one
    HIP graph and replayed between two events, so the figure is the kernels'
    own time back to back, not the host's per-call binding overhead (which
    exceeds these kernels' few microseconds when they are launched from
    Python one by one)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_.record(cur)
    g.replay()
    b_.record(cur)
    torch.cuda.synchronize()
    return round(a_.elapsed_time(b_) / iters * 1e3, 2)


def generate_host(w):
    """Full logits of every request on the host: target row (r, j) at r*(K+1) + j,
    draft row (r, j) at r*K + j (NaN elsewhere), and both modes' draft ids."""
    n, K, V = w.n, w.k_max, w.vocab
    tgt_full = np.full((n * (K + 1), V), np.nan, dtype=np.float32)
    drf_full = np.full((n * K, V), np.nan, dtype=np.float32)
    toks = {m: np.full((n, K), -1, dtype=np.int32) for m in ("stochastic", "greedy")}
    for r in range(n):
        rq = w.request(r)
        Kr = int(w.draft_len[r])
        tgt_full[r * (K + 1): r * (K + 1) + Kr + 1] = rq["target"]
        drf_full[r * K: r * K + Kr] = rq["draft"]
        toks["stochastic"][r] = rq["tok_stochastic"]
        toks["greedy"][r] = rq["tok_greedy"]
        w.drop_cache()
    return tgt_full, drf_full, toks


def generate_device(torch, w, ldt):
    """The same layout as generate_host, written to the device request by request
    (the large workloads never sit whole in host memory); padding rows are NaN."""
    n, K, V = w.n, w.k_max, w.vocab
    dev = torch.device("cuda:0")
    tgt = torch.full((n * (K + 1), V), float("nan"), dtype=ldt, device=dev)
    drf = torch.full((n * K, V), float("nan"), dtype=ldt, device=dev)
    toks = {m: np.full((n, K), -1, dtype=np.int32) for m in ("stochastic", "greedy")}
    for r in range(n):
        rq = w.request(r)
        Kr = int(w.draft_len[r])
        tgt[r * (K + 1): r * (K + 1) + Kr + 1] = torch.from_numpy(rq["target"]).to(dev, ldt)
        if Kr:
            drf[r * K: r * K + Kr] = torch.from_numpy(rq["draft"]).to(dev, ldt)
        toks["stochastic"][r] = rq["tok_stochastic"]
        toks["greedy"][r] = rq["tok_greedy"]
        w.drop_cache()
    torch.cuda.synchronize()
    return tgt, drf, toks


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); the verify step would shard by request with "
              f"no exchange.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return

    import torch

    import adaptive_draft_verification_amd as sv
    import workloads

    w = workloads.make(args.workload)
    ldt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    n, K, V = w.n, w.k_max, w.vocab

    t0 = time.time()
    tgt_full, drf_full, toks_all = generate_host(w)
    toks_np = toks_all[args.mode]
    print(f"[bench] generated {args.workload} in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    # the CPU oracle first: its worker processes fork before the GPU is touched
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, w, tgt_full, drf_full, toks_np)
        print(f"[bench] cpu baseline: {cpu['value']} rows/s on {cpu['cores']} workers",
              file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def d(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.to(dtype) if dtype is not None else t).to(dev)

    tgt_full_d = d(tgt_full, ldt)
    drf_full_d = d(drf_full, ldt)
    del tgt_full, drf_full
    leg = Leg(sv, torch, w, args.mode, tgt_full_d, drf_full_d, toks_np, args)
    if args.all_drafts:
        # verify reads every draft's rows; the step's budget and pack still run
        reps_all, cu_all, rows_ta, rows_da = leg.full_k_inputs()
        leg.replicas, leg.verify_cu = reps_all, cu_all
        leg.rows_t, leg.rows_d, leg.B = rows_ta, int(w.draft_len.sum()), int(w.draft_len.sum())
        leg.kept_h = w.draft_len.copy()
    mode = leg.mode
    rows_t, rows_d, B = leg.rows_t, leg.rows_d, leg.B
    esize = leg.esize

    # the headline: K steps back to back, launched eagerly or replayed from HIP
    # graphs (one per replica and Philox step, cycled)
    graphs = []
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(2):
                leg.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(args.graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                leg.step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(i):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            leg.step(i)

    for i in range(args.warmup):
        run_step(i)
    wall = timed_plain(torch, args.steps, run_step)
    wall_eager = timed_plain(torch, args.steps, leg.step) if graphs else wall
    step_pct = step_percentiles(torch, leg.stream, args.steps, run_step)
    # per-stage times in a separate loop (events between stages cost time)
    for i in range(2):
        leg.step(i)
    _, stage_ms = leg.timed(args.steps)
    p2_ids = leg.pass2_ids(range(args.steps), leg.kept_h)

    ms_per_step = wall * 1e3 / args.steps
    pass1_ms, pass2_ms = float(np.mean(stage_ms[:, 2])), float(np.mean(stage_ms[:, 3]))
    verify_us = (stage_ms[:, 2] + stage_ms[:, 3]) * 1e3
    roof_ms = leg.pass1_launch_ms(args.steps)
    verify_ms = leg.verify_launch_ms(args.steps)
    pass1_bytes = leg.pass1_bytes(rows_t, rows_d)
    pass2_bytes = float(np.mean(p2_ids)) * esize
    achieved = pass1_bytes / (roof_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- full K leg
    full = None
    if args.full_k_iters > 0:
        full_reps, cu_full, rows_tf, rows_df = leg.full_k_inputs()
        kw = dict(reps=full_reps, cu_rows=cu_full, kept_in=True)
        for i in range(3):
            leg.step(i, **kw)
        _, fms = leg.timed(args.full_k_iters, **kw)
        f1, f2 = float(np.mean(fms[:, 2])), float(np.mean(fms[:, 3]))
        f_p1 = leg.pass1_bytes(rows_tf, rows_df)
        f_p2 = float(np.mean(leg.pass2_ids(range(args.full_k_iters), w.draft_len, **kw))) \
            * esize
        f1_launch = leg.pass1_launch_ms(args.full_k_iters, reps=full_reps, cu_rows=cu_full)
        full = {
            "target_rows": rows_tf, "draft_rows": rows_df,
            "pass1_us": round(f1 * 1e3, 2), "pass2_us": round(f2 * 1e3, 2),
            "pass1_launch_us": round(f1_launch * 1e3, 2),
            "pass1_bytes": int(f_p1), "pass2_bytes": int(f_p2),
            "pass1_gbps": round(f_p1 / (f1_launch * 1e-3) / 1e9, 1),
            "pass1_frac": round(f_p1 / (f1_launch * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "pass2_gbps": round(f_p2 / (f2 * 1e-3) / 1e9, 1) if f_p2 else None,
            "verify_gbps": round((f_p1 + f_p2) / ((f1 + f2) * 1e-3) / 1e9, 1),
            "verify_frac": round((f_p1 + f_p2) / ((f1 + f2) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "verify_rows_per_s": round(rows_tf / ((f1 + f2) * 1e-3), 1),
            "iters": args.full_k_iters,
        }
        del full_reps

    # -------------------------------------------- draft-row features leg
    # pass 1 asked for the draft rows' entropy and largest probability as well
    features = None
    if mode == sv.SV_STOCHASTIC:
        feat_ms = leg.pass1_launch_ms(args.steps, features=True)
        features = {"pass1_us": round(feat_ms * 1e3, 2),
                    "pass1_gbps": round(pass1_bytes / (feat_ms * 1e-3) / 1e9, 1),
                    "vs_plain_pass1": round(feat_ms / roof_ms, 4)}

    # ------------------------------------------------ uniform draft length leg
    # the DSD-style alternative to the adaptive budget: one K for the batch
    conf_d, dl_d, cost_d, last_d, toks_d = leg.conf_d, leg.dl_d, leg.cost_d, leg.last_d, leg.toks_d
    err, bws, cap = leg.err, leg.bws, leg.cap
    uk_k = torch.empty(1, dtype=torch.int32, device=dev)
    uk_kept = torch.empty(n, dtype=torch.int32, device=dev)
    small_iters = max(SMALL_CALL_ITERS, args.steps)
    uk_us = graph_us(torch, lambda: sv.sv_uniform_k_select(conf_d, dl_d, cost_d, w.t_base,
                                                           w.n_bonus, uk_kept, uk_k, None, err),
                     small_iters)
    uniform_k = {"us": uk_us, "k": int(uk_k.item()), "drafts_verified": int(uk_kept.sum().item())}

    # the step's budget and pack call on its own, graph-replayed: its kernels'
    # time without the staged loop's events around it
    bs_kept = torch.empty(n, dtype=torch.int32, device=dev)
    bs_budget = torch.empty(1, dtype=torch.int32, device=dev)
    bs_cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
    bs_maps = [torch.empty(cap, dtype=torch.int32, device=dev) for _ in range(3)]
    budget_select_graph_us = graph_us(
        torch,
        lambda: sv.sv_budget_select_pack(conf_d, dl_d, cost_d, w.t_base, w.n_bonus, last_d,
                                         toks_d, bs_kept, bs_budget, bs_cu, *bs_maps, None, err,
                                         ws=bws),
        small_iters)
    # and the two calls it fuses, each on its own
    budget_only_graph_us = graph_us(
        torch,
        lambda: sv.sv_budget_select(conf_d, dl_d, cost_d, w.t_base, w.n_bonus, bs_kept,
                                    bs_budget, None, err, ws=bws),
        small_iters)
    pack_graph_us = graph_us(
        torch,
        lambda: sv.sv_pack_varlen(bs_kept, last_d, toks_d, bs_cu, *bs_maps, err),
        small_iters)

    # ----------------------------------------- stale-confidence budget leg
    # the pipeline that sizes B one step ahead: the step itself only allocates
    # the slots of a B already in device memory (here the budget selected above)
    al_kept = torch.empty(n, dtype=torch.int32, device=dev)
    budget_allocate_us = graph_us(
        torch, lambda: sv.sv_budget_allocate(conf_d, dl_d, leg.budget, al_kept, None, None, err,
                                             ws=bws),
        small_iters)

    # ------------------------------------------ acceptance statistics and calibration leg
    # one verify with the draft-row features, then the per-position counters and
    # one update and prediction of the logistic acceptance model from its outcome
    calibration = None
    if mode == sv.SV_STOCHASTIC:
        qh = torch.empty(n, K, dtype=torch.float32, device=dev)
        qm = torch.empty(n, K, dtype=torch.float32, device=dev)
        tp0, dr0 = leg.replicas[0]
        sv.sv_verify_stages(tp0, dr0, toks_d, leg.cu, mode, w.tau, w.seed, 0, leg.tok_out,
                            leg.acc_out, leg.ws, 3, leg.p_out, leg.q_out, leg.res_out, err,
                            vocab=V, out_q_entropy=qh, out_q_max=qm)
        attempted = torch.zeros(K, dtype=torch.int64, device=dev)
        accepted_at = torch.zeros(K, dtype=torch.int64, device=dev)
        totals = torch.zeros(2, dtype=torch.int64, device=dev)
        theta = torch.zeros(K + 3, dtype=torch.float32, device=dev)
        pred = torch.empty(n, K, dtype=torch.float32, device=dev)
        legs = {
            "accept_stats_us": lambda: sv.sv_accept_stats(leg.acc_out, leg.cu, attempted,
                                                          accepted_at, totals),
            "calibrate_update_us": lambda: sv.sv_calibrate_update(
                theta, leg.q_out, leg.acc_out, leg.cu, 1e-3, q_entropy=qh, q_max=qm),
            "calibrate_predict_us": lambda: sv.sv_calibrate_predict(
                theta, leg.q_out, pred, q_entropy=qh, q_max=qm),
        }
        calibration = {key: graph_us(torch, fn, small_iters) for key, fn in legs.items()}

    # ---------------------------------- greedy mode on the same workload
    # (same logit replicas and budget; the drafter's argmax ids; pass 1 reads
    # the target rows only and pass 2 draws nothing)
    wanted = set(x for x in args.legs.split(",") if x and x != "none")
    greedy = None
    if "greedy" in wanted and mode == sv.SV_STOCHASTIC:
        gleg = Leg(sv, torch, w, "greedy", tgt_full_d, drf_full_d, toks_all["greedy"], args,
                   share=leg)
        greedy = gleg.leg_figures(args.steps, args.full_k_iters)
        del gleg
        print(f"[bench] greedy leg: {greedy['step_us']} us/step", file=sys.stderr, flush=True)

    # ----------------------------- the mixed-length fp32 workload (V = 256,000)
    mix = None
    if "mix" in wanted:
        del leg.replicas, tgt_full_d, drf_full_d
        torch.cuda.empty_cache()
        t1 = time.time()
        wm = workloads.make("b256_mix_v256000")
        mldt = torch.bfloat16 if wm.dtype == "bf16" else torch.float32
        mt, md, mtoks = generate_device(torch, wm, mldt)
        print(f"[bench] generated {wm.name} in {time.time() - t1:.1f}s", file=sys.stderr,
              flush=True)
        mleg = Leg(sv, torch, wm, "stochastic", mt, md, mtoks["stochastic"], args)
        del mt, md
        mix = mleg.leg_figures(max(10, args.steps // 4), max(10, args.full_k_iters // 4)
                               if args.full_k_iters > 0 else 0)
        del mleg
        torch.cuda.empty_cache()
        print(f"[bench] mixed leg: {mix['step_us']} us/step", file=sys.stderr, flush=True)

    traffic = None if args.all_drafts else measured_traffic(args.workload, args.mode)
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
            "cost_granule": w.granule, "drafts": "all" if args.all_drafts else "adaptive",
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "rowstats_kernel (verify pass 1)",
                     "bytes_per_launch": int(pass1_bytes),
                     "launch_us": round(roof_ms * 1e3, 2)},
        "budget_pack": "separate" if args.separate_pack else "fused",
        "budget_select_us": round(float(np.mean(stage_ms[:, 0])) * 1e3, 2),
        "budget_select_graph_us": budget_select_graph_us,
        "budget_select_only_graph_us": budget_only_graph_us,
        "pack_varlen_graph_us": pack_graph_us,
        "small_call_iters": small_iters,
        "budget_allocate_us": budget_allocate_us,
        "pack_us": round(float(np.mean(stage_ms[:, 1])) * 1e3, 2),
        "verify_pass1_us": round(pass1_ms * 1e3, 2),
        "verify_pass2_us": round(pass2_ms * 1e3, 2),
        "verify_pass2_bytes": int(pass2_bytes),
        "verify_pass2_frac": (round(pass2_bytes / (pass2_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                              if pass2_bytes else None),
        # the verify step alone (both passes, from the staged loop's events)
        "verify_us_p10_p50_p90": [round(float(np.percentile(verify_us, q)), 2)
                                  for q in (10, 50, 90)],
        "verify_rows_per_s": round(rows_t / (float(np.median(verify_us)) * 1e-6), 1),
        "verify_gbps": round((pass1_bytes + pass2_bytes)
                             / (float(np.median(verify_us)) * 1e-6) / 1e9, 1),
        "verify_frac": round((pass1_bytes + pass2_bytes) / (float(np.median(verify_us)) * 1e-6)
                             / 1e9 / HBM_PEAK_GBPS, 4),
        # the same call timed back to back, no event between its two passes
        "verify_launch_us": round(verify_ms * 1e3, 2),
        "verify_launch_frac": round((pass1_bytes + pass2_bytes) / (verify_ms * 1e-3) / 1e9
                                    / HBM_PEAK_GBPS, 4),
        "gpu_step_us": round(float(np.mean(stage_ms.sum(axis=1))) * 1e3, 2),
        "launch": "hip-graph replay" if graphs else "eager",
        "step_us_p10_p50_p90": step_pct,
        "ms_per_step_eager": round(wall_eager * 1e3 / args.steps, 4),
        "step_hbm_gbps": round((pass1_bytes + pass2_bytes) / (ms_per_step * 1e-3) / 1e9, 1),
        "uniform_k": uniform_k,
        "calibration": calibration,
        "draft_features": features,
        "full_k": full,
        "greedy": greedy,
        "mix_v256000": mix,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
