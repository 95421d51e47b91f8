"""Planted-mistake check of the oracle's pins (run by hand, CPU only).

    python tests/oracle_mutations.py [-j JOBS] [NAME ...]

Each entry below plants one plausible slip in a scratch copy of oracle/ — a
sign, an operand order, an index off by one, a missing break, a reversed tie
rule, fp64 where fp32 is fixed, round for floor, a missing mean, a dropped
clamp, swapped Philox counter words — and runs the CPU tests on that copy
(without the two statistical tests, which take most of the suite's time).
A slip that no test notices is printed as SURVIVED and makes the exit status
1.  The unmodified copy is run first and must pass.  Nothing here touches the
repository itself.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# what the CPU tests read (the built library stays out: the tests that need it skip)
KEEP = ("oracle", "tests", "workloads", "include", "adaptive_draft_verification_amd",
        "pytest.ini")
SKIP = ("__pycache__", "*.so")
PYTEST = ["-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
          "-k", "not chi_square and not uniformity",
          "--ignore=tests/test_gpu_parity.py", "--ignore=tests/test_zz_no_alloc.py",
          "--ignore=tests/test_abi.py"]

# (file under oracle/, text replaced, replacement, name)
M = [
 # verify
 ("verify.py", "/ float(tau)\n    y = y - y.max()", "* float(tau)\n    y = y - y.max()", "row_probs z*tau"),
 ("verify.py", "        return p_d > 0.0", "        return True", "q=0 always accepts"),
 ("verify.py", "        return p_d > 0.0", "        return False", "q=0 always rejects"),
 ("verify.py", "    return u < p_d / q_d", "    return u < q_d / p_d if p_d > 0 else False", "ratio inverted"),
 ("verify.py", "    return u < p_d / q_d", "    return u > p_d / q_d", "accept sign flipped"),
 ("verify.py", "np.maximum(0.0, p - q)", "np.maximum(0.0, q - p)", "residual q-p"),
 ("verify.py", "np.maximum(0.0, p - q)", "np.abs(p - q)", "residual abs"),
 ("verify.py", "        return p.copy(), mass", "        return np.ones_like(p), mass", "zero-mass fallback uniform"),
 ("verify.py", "    hit = np.nonzero(c > t)[0]", "    hit = np.nonzero(c >= t)[0]", "cdf >="),
 ("verify.py", "    t = v * c[-1]", "    t = v", "cdf unnormalised"),
 ("verify.py", "    return int(np.nonzero(w > 0)[0][-1])", "    return len(w) - 1", "no-hit last id"),
 ("verify.py", "        w = p[b]\n", "        w = p[b - 1] if b > 0 else p[b]\n", "bonus from row b-1"),
 ("verify.py", "    _, v = uniforms(seed, r, L, step)", "    _, v = uniforms(seed, r, L + 1, step)", "draw counter L+1"),
 ("verify.py", "    _, v = uniforms(seed, r, L, step)", "    v, _ = uniforms(seed, r, L, step)", "draw uses u"),
 ("verify.py", "        u, _ = uniforms(seed, r, j, step)", "        _, u = uniforms(seed, r, j, step)", "accept uses v"),
 ("verify.py", "            natural = j\n            break", "            natural = j", "last rejection"),
 ("verify.py", "        pd, qd = float(p[j][d]), float(q[j][d])", "        qd, pd = float(p[j][d]), float(q[j][d])", "p/q swapped"),
 ("verify.py", "        pd, qd = float(p[j][d]), float(q[j][d])", "        pd, qd = float(p[j + 1][d]), float(q[j][d])", "target row off by one"),
 ("verify.py", "            if int(dtoks[j]) != argmaxes[j]:", "            if int(dtoks[j]) != argmaxes[j + 1]:", "greedy row off by one"),
 ("verify.py", "    return int(np.argmax(z))", "    return int(len(z) - 1 - np.argmax(z[::-1]))", "argmax last tie"),
 ("verify.py", "np.isneginf(z).all())", "np.isneginf(z).any())", "fault on any -inf"),
 ("verify.py", "    return bool(np.isnan(z).any() or np.isposinf(z).any() or np.isneginf(z).all())", "    return bool(np.isnan(z).any() or np.isneginf(z).all())", "+inf not a fault"),
 ("verify.py", "    out[\"tokens\"] = [int(d) for d in dtoks[:L]] + [tok]", "    out[\"tokens\"] = [int(d) for d in dtoks[:L]] + [tok if L < b else int(np.argmax(w))]", "bonus argmax"),
 ("verify.py", "        if lo < 0 or b < 0 or b > k_max or hi > rows_avail:", "        if lo < 0 or b < 0 or hi > rows_avail:", "no k_max check"),
 # features
 ("features.py", "    y = y / float(tau)", "    y = y * float(tau)", "features z*tau"),
 ("features.py", "np.log2(pos)", "np.log(pos)", "entropy nats"),
 ("features.py", "    return entropy, float(q.max())", "    return entropy, float(e.max())", "max unnormalised"),
 # budget
 ("budget.py", "    if np.isnan(c) or c <= 0:", "    if np.isnan(c) or c < 0:", "clamp keeps -0"),
 ("budget.py", "    if c > 1:\n        return np.float32(1.0)", "    if c > 1:\n        return c", "no clamp above 1"),
 ("budget.py", "            prev = np.float32(prev * clamp_confidence(conf[r, j]))", "            prev = np.float32(clamp_confidence(conf[r, j]))", "no running product"),
 ("budget.py", "            prev = np.float32(prev * clamp_confidence(conf[r, j]))", "            prev = np.float64(prev) * np.float64(clamp_confidence(conf[r, j]))", "survival in fp64"),
 ("budget.py", "        if raw[t] > m:", "        if raw[t] < m:", "running min"),
 ("budget.py", "        padded = ((t + granule - 1) // granule) * granule", "        padded = (t // granule) * granule", "pad down"),
 ("budget.py", "key=lambda rj: (-float(s[rj[0], rj[1]]), rj[0], rj[1])", "key=lambda rj: (-float(s[rj[0], rj[1]]), -rj[0], rj[1])", "ties higher request"),
 ("budget.py", "    return int(math.floor(float(sv) * (2.0 ** FIXED_SHIFT)))", "    return int(round(float(sv) * (2.0 ** FIXED_SHIFT)))", "fixed round"),
 ("budget.py", "    return (float(n_bonus) + float(s_fixed) * (2.0 ** -FIXED_SHIFT)) / c", "    return (float(s_fixed) * (2.0 ** -FIXED_SHIFT)) / c", "no bonus"),
 ("budget.py", "        cval = float(cost[t_base + b])", "        cval = float(cost[b])", "cost ignores t_base"),
 ("budget.py", "        cval = float(cost[t_base + b])", "        cval = float(cost[t_base + b + 1])", "cost off by one"),
 ("budget.py", "        if best is None or sc > best:", "        if best is None or sc >= best:", "ties largest B"),
 ("budget.py", "    used = min(max(int(budget), 0), len(order))", "    used = min(abs(int(budget)), len(order))", "negative B abs"),
 # pack
 ("pack.py", "        cu_rows[r + 1] = cu_rows[r] + b[r] + 1", "        cu_rows[r + 1] = cu_rows[r] + b[r]", "rows no +1"),
 ("pack.py", "else int(draft_tokens[r, i - 1])", "else int(draft_tokens[r, i])", "draft token off by one"),
 ("pack.py", "            row_pos[row] = i", "            row_pos[row] = i + 1", "row_pos shifted"),
 # philox
 ("philox.py", "        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0", "        c0, c1, c2, c3 = (hi0 ^ c1 ^ k0), lo1, (hi1 ^ c3 ^ k1), lo0", "philox hi swapped"),
 ("philox.py", "PHILOX_ROUNDS = 10", "PHILOX_ROUNDS = 7", "philox 7 rounds"),
 ("philox.py", "    v = (x1 >> np.uint64(8)).astype(np.float64) * scale", "    v = (x1 >> np.uint64(9)).astype(np.float64) * (2 * scale)", "v 23 bits"),
 ("philox.py", "(request, position, step & 0xFFFFFFFF, step >> 32,", "(position, request, step & 0xFFFFFFFF, step >> 32,", "counter order"),
 # uniform_k
 ("uniform_k.py", "            m = min(K, int(lens[r]))", "            m = K", "uniform K ignores draft_len"),
 ("uniform_k.py", "        cval = float(cost[t_base + t])", "        cval = float(cost[t_base + K])", "uniform K cost per K"),
 ("uniform_k.py", "        if best is None or sc > best:", "        if best is None or sc >= best:", "uniform K ties largest"),
 # calibrate
 ("calibrate.py", "    return min(0.0, max(X_MIN, math.log2(q)))", "    return min(0.0, max(X_MIN, math.log(q)))", "feature ln"),
 ("calibrate.py", "            for j in range(min(L, b - 1) + 1 if b > 0 else 0):", "            for j in range(min(L, b) if b > 0 else 0):", "rejected position dropped"),
 ("calibrate.py", "                obs.append((j, 1 if j < L else 0))", "                obs.append((j, 1 if j <= L else 0))", "label off by one"),
 ("calibrate.py", "            err = sigmoid(_logit(theta, k_max, j, x)) - y", "            err = y - sigmoid(_logit(theta, k_max, j, x))", "gradient sign"),
 ("calibrate.py", "        theta -= lr * g / count", "        theta -= lr * g", "no mean"),
 ("calibrate.py", "        emitted += L + 1", "        emitted += L", "emitted no bonus"),
 ("calibrate.py", "    return min(H_MAX, h) if h > 0 else 0.0", "    return min(H_MAX, h) if h > 0 else -1.0", "entropy negative reads -1"),
 ("verify.py", "                L = j\n                break", "                L = j", "greedy last mismatch"),
 ("verify.py", "    q = [row_probs(drows[j], tau) for j in range(b)]", "    q = [row_probs(trows[j], tau) for j in range(b)]", "q from target rows"),
 ("features.py", "    entropy = float(-(pos * np.log2(pos)).sum()) + 0.0", "    entropy = float((pos * np.log2(pos)).sum()) + 0.0", "entropy sign"),
 ("calibrate.py", "    return min(0.0, max(X_MIN, math.log2(q)))", "    return min(0.0, math.log2(q))", "feature unclamped"),
 ("calibrate.py", "            0.0 if q_entropy is None else entropy_feature(q_entropy[r, j]),\n            0.0 if q_max is None else max_feature(q_max[r, j]))", "            0.0 if q_max is None else max_feature(q_max[r, j]),\n            0.0 if q_entropy is None else entropy_feature(q_entropy[r, j]))", "features swapped"),
 ("uniform_k.py", "    kept = np.minimum(lens, best_k).astype(np.int32)", "    kept = np.full(n, best_k).astype(np.int32)", "uniform K kept ignores lens"),
 ("budget.py", "    for r, _j in order[:best_b]:", "    for r, _j in order[:best_b + 1]:", "kept one extra"),
 ("budget.py", "        out[t] = running[padded]", "        out[t] = raw[padded]", "cost not monotone"),
 ("pack.py", "            packed[row] = int(last_token[r]) if i == 0 else int(draft_tokens[r, i - 1])", "            packed[row] = int(draft_tokens[r, i - 1]) if i > 0 else -1", "pack drops last token"),
]


def run(entry, scratch):
    f, old, new, name = entry
    d = tempfile.mkdtemp(dir=scratch)
    try:
        dst = os.path.join(d, "repo")
        os.makedirs(dst)
        for item in KEEP:
            src = os.path.join(ROOT, item)
            if os.path.isdir(src):
                shutil.copytree(src, os.path.join(dst, item),
                                ignore=shutil.ignore_patterns(*SKIP))
            elif os.path.exists(src):
                shutil.copy2(src, os.path.join(dst, item))
        if old is not None:
            path = os.path.join(dst, "oracle", f)
            text = open(path).read()
            if text.count(old) != 1:
                return name, "ANCHOR NOT FOUND", ""
            open(path, "w").write(text.replace(old, new))
        r = subprocess.run([sys.executable, *PYTEST], cwd=dst, capture_output=True, text=True,
                           timeout=900)
        last = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else r.stderr[-200:]
        if old is None:
            return name, "PASSED" if r.returncode == 0 else "FAILED", last
        # a failure must come from a test, not from collection
        caught = r.returncode == 1 and " failed" in last
        return name, "CAUGHT" if caught else "SURVIVED", last
    finally:
        shutil.rmtree(d, ignore_errors=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=6)
    ap.add_argument("names", nargs="*")
    a = ap.parse_args()
    todo = [m for m in M if not a.names or m[3] in a.names]
    bad = 0
    with tempfile.TemporaryDirectory() as scratch:
        name, status, last = run(("", None, None, "unmodified oracle"), scratch)
        print(f"{name} | {status} | {last}", flush=True)
        if status != "PASSED":
            return 1
        with cf.ThreadPoolExecutor(a.j) as ex:
            for name, status, last in ex.map(lambda m: run(m, scratch), todo):
                print(f"{name} | {status} | {last}", flush=True)
                bad += status != "CAUGHT"
    print(f"{len(todo) - bad} of {len(todo)} caught")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
