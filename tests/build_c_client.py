"""Build tests/c_gpu_client (a plain C caller of the library on a GPU) next to
its source.  Called by __graft_entry__.build() after the library, so that the
GPU test finds it built; run by hand with `python tests/build_c_client.py`."""

import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_gpu_client.c")
EXE = os.path.join(ROOT, "tests", "c_gpu_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler to build tests/c_gpu_client")
    cmd = [cc, "-std=gnu11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "adaptive_draft_verification_amd"), "-l:libspecverify.so",
           "-Wl,-rpath,$ORIGIN/../adaptive_draft_verification_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building tests/c_gpu_client failed:\n" + r.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
