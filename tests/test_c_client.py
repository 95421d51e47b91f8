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
