"""The header as a C header: a plain C program (tests/c_abi_client.c) compiles
against include/libspecverify.h as C99 and as C11 with -pedantic -Werror,
links against libspecverify.so, and its host-only calls return what the
binding and the oracle say.  Nothing here touches a device."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sv = pytest.importorskip("adaptive_draft_verification_amd",
                         reason="libspecverify.so not built (python adaptive_draft_verification_amd/build.py)")
GCC = shutil.which("gcc")


def build_and_run(std, tmp_path):
    lib_dir = os.path.dirname(sv.LIB_PATH)
    exe = str(tmp_path / f"c_abi_client_{std}")
    rocm_lib = "/opt/rocm/lib"
    cmd = [GCC, f"-std={std}", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"),
           "-o", exe, "-L", lib_dir, "-l:libspecverify.so", f"-Wl,-rpath,{lib_dir}",
           f"-Wl,-rpath-link,{rocm_lib}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, _, rest = line.partition(" ")
        if key == "status":
            code, _, text = rest.partition(" ")
            out[f"status{code}"] = text
        else:
            out[key] = rest
    return out


@pytest.mark.skipif(GCC is None, reason="no C compiler")
@pytest.mark.parametrize("std", ["c99", "c11"])
def test_plain_c_client(std, tmp_path):
    out = build_and_run(std, tmp_path)
    for s in range(9):
        assert out[f"status{s}"] == sv.sv_status_str(s)
    assert int(out["budget_ws"]) == sv.sv_budget_workspace_bytes(256, 7)
    assert int(out["verify_ws"]) == sv.sv_verify_workspace_bytes(256, 7)
    assert int(out["verify_ws_refused"]) == 0
    assert int(out["cost_status"]) == sv.SV_OK
    raw = np.array([1, 3, 2, 5, 4, 4.5, 7, 6, 8], dtype=np.float32)
    want = oracle.cost_table_prepare(raw, 2, 7)
    got = np.array([float(x) for x in out["cost"].split()], dtype=np.float32)
    np.testing.assert_array_equal(got, np.asarray(want, dtype=np.float32))
    assert int(out["cost_bad_value"]) == sv.SV_ERR_VALUE
    assert int(out["cost_null"]) == sv.SV_ERR_NULL
    assert int(out["budget_null"]) == sv.SV_ERR_NULL
    assert int(out["pack_shape"]) == sv.SV_ERR_SHAPE
    assert int(out["verify_dtype"]) == sv.SV_ERR_DTYPE
    assert int(out["verify_temperature"]) == sv.SV_ERR_VALUE
    assert int(out["verify_nothing"]) == sv.SV_OK
    assert int(out["noalloc_capacity"]) == sv.SV_ERR_CAPACITY


EXE = os.path.join(ROOT, "tests", "c_gpu_client")


@pytest.mark.gpu
def test_plain_c_client_on_the_gpu(tmp_path):
    """The whole path driven from C through the ABI alone (tests/c_gpu_client.c):
    budget and packing in one call, the target rows gathered into the packed
    layout, stochastic verification; every output against the oracle."""
    from parity import compare_verify

    if not os.path.exists(EXE):
        pytest.skip("tests/c_gpu_client not built (python tests/build_c_client.py)")
    rng = np.random.default_rng(4242)
    n, k, V, tau, seed, step = 8, 4, 3001, 0.8, 7, 11
    conf = (rng.beta(8, 2, (n, k)) ** np.arange(1, k + 1)).astype(np.float32)
    draft_len = rng.integers(1, k + 1, n).astype(np.int32)
    t_base = n_bonus = n
    t = np.arange(n * (k + 1) + 1)
    raw = np.maximum(1.0, t / 16.0).astype(np.float32)
    cost = np.asarray(oracle.cost_table_prepare(raw, 4, len(raw)), dtype=np.float32)
    last_token = rng.integers(0, V, n).astype(np.int32)
    target = (rng.standard_normal((n * (k + 1), V)) * 3).astype(np.float32)
    draft = np.empty((n * k, V), dtype=np.float32)
    toks = np.empty((n, k), dtype=np.int32)
    for r in range(n):
        for j in range(k):
            row = target[r * (k + 1) + j] + rng.standard_normal(V).astype(np.float32)
            draft[r * k + j] = row
            toks[r, j] = int(np.argmax(row / tau - np.log(rng.standard_exponential(V))))
    (tmp_path / "meta.txt").write_text(
        f"{n} {k} {V} {len(cost)} {t_base} {n_bonus} {seed} {step} {tau!r}\n")
    for name, arr in (("conf.f32", conf), ("draft_len.i32", draft_len), ("cost.f32", cost),
                      ("last_token.i32", last_token), ("draft_tokens.i32", toks),
                      ("target.f32", target), ("draft.f32", draft)):
        arr.tofile(str(tmp_path / name))
    print(f"c client: n={n} k={k} V={V} tau={tau}", flush=True)
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, _, rest = line.partition(" ")
        out[key] = rest.split()

    ob = oracle.budget_select(conf, draft_len, k, cost, t_base, n_bonus)
    assert int(out["budget"][0]) == ob["budget"]
    assert int(out["budget_dev_error"][0]) == ob["dev_error"]
    kept = np.array(out["kept"], dtype=np.int64)
    np.testing.assert_array_equal(kept, ob["kept"])
    op = oracle.pack_varlen(ob["kept"], last_token, toks, k)
    cu = np.array(out["cu_rows"], dtype=np.int32)
    np.testing.assert_array_equal(cu, op["cu_rows"])

    packed = np.concatenate([target[r * (k + 1): r * (k + 1) + int(kept[r]) + 1]
                             for r in range(n)])
    g = {"tokens": np.array(out["tokens"], dtype=np.int32).reshape(n, k + 1),
         "accepted": np.array(out["accepted"], dtype=np.int32),
         "p_draft": np.array(out["p_draft"], dtype=np.float32).reshape(n, k),
         "q_draft": np.array(out["q_draft"], dtype=np.float32).reshape(n, k),
         "residual_mass": np.array(out["residual_mass"], dtype=np.float32),
         "dev_error": np.array(out["verify_dev_error"], dtype=np.int32)}
    compare_verify(g, packed, draft, toks, cu, k, V, "stochastic", tau, seed, step)
