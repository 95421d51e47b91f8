"""Pins for the oracle's Philox4x32-10 (CPU only).

1. Bit equality with a second, independent implementation: rocRAND's
   host-callable Philox4x32-10 engine, built here from its public header.
   rocRAND's state after rocrand_init(seed, subsequence, offset) uses key =
   seed and counter = (offset / 4 as a 64-bit number, subsequence as a 64-bit
   number), so counter (r, j, step_lo, step_hi) is offset 4 * (r + j * 2**32)
   of subsequence `step`.
2. Uniformity of u and v (chi-square and Kolmogorov-Smirnov) and independence
   of u from v (2-D chi-square) over 10**7 counters.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND host reference")
    out = tmp_path_factory.mktemp("philox") / "philox_ref"
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-o", str(out),
           os.path.join(HERE, "philox_rocrand_ref.cpp")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("could not build rocRAND reference: " + res.stderr[-400:])
    return str(out)


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(5)
    cases = []
    for i in range(3000):
        seed = int(rng.integers(0, 2**63)) if i % 3 else int(rng.integers(0, 2**16))
        r = int(rng.integers(0, 2**32)) if i % 5 == 0 else int(rng.integers(0, 4096))
        j = int(rng.integers(0, 2**30)) if i % 7 == 0 else int(rng.integers(0, 64))
        step = int(rng.integers(0, 2**63)) if i % 2 else int(rng.integers(0, 1000))
        cases.append((seed, r, j, step))
    cases += [(0, 0, 0, 0), (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**64 - 1)]
    lines = "".join(f"{s} {st} {4 * (r + (j << 32))}\n" for s, r, j, st in cases)
    res = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True)
    ref = np.array([[int(x) for x in ln.split()] for ln in res.stdout.strip().splitlines()],
                   dtype=np.uint64)
    seeds = np.array([c[0] for c in cases], dtype=np.uint64)
    rs = np.array([c[1] for c in cases], dtype=np.uint64)
    js = np.array([c[2] for c in cases], dtype=np.uint64)
    steps = np.array([c[3] for c in cases], dtype=np.uint64)
    m = np.uint64(0xFFFFFFFF)
    got = oracle.philox4x32_10(rs, js, steps & m, steps >> np.uint64(32),
                               seeds & m, seeds >> np.uint64(32))
    got = np.stack(got, axis=1)
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got, ref)


def test_uniforms_follow_the_rocrand_stream(rocrand_ref):
    """u and v of (request r, position j, step) are the top 24 bits of words 0
    and 1 of the block at offset 4 * (r + j * 2**32) of rocRAND's Philox
    subsequence `step` under the seed, each scaled by 2**-24."""
    rng = np.random.default_rng(6)
    cases = [(int(rng.integers(0, 2**63)), int(rng.integers(0, 5000)), int(rng.integers(0, 16)),
              int(rng.integers(0, 2**40))) for _ in range(500)]
    cases += [(0, 0, 0, 0), (1, 2, 3, 4), (2**64 - 1, 2**32 - 1, 15, 2**64 - 1)]
    lines = "".join(f"{s} {st} {4 * (r + (j << 32))}\n" for s, r, j, st in cases)
    res = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True)
    words = [[int(x) for x in ln.split()] for ln in res.stdout.strip().splitlines()]
    assert len(words) == len(cases)
    for (seed, r, j, step), w in zip(cases, words):
        u, v = oracle.uniforms(seed, r, j, step)
        assert u == (w[0] >> 8) / 2**24 and v == (w[1] >> 8) / 2**24, (seed, r, j, step)


def test_uniforms_are_24_bit_grid_values():
    u, v = oracle.uniforms(123, np.arange(1000), 3, 9)
    for x in (u, v):
        assert np.all((x >= 0) & (x < 1))
        np.testing.assert_array_equal(x * 2**24, np.floor(x * 2**24))
    # scalars give the same numbers as arrays
    us, vs = oracle.uniforms(123, 17, 3, 9)
    assert us == u[17] and vs == v[17]


def test_uniformity_and_independence():
    n = 10**7
    r = np.arange(n, dtype=np.uint64) % np.uint64(65536)
    j = np.arange(n, dtype=np.uint64) // np.uint64(65536)
    u, v = oracle.uniforms(20261202, r, j, 77)
    for x in (u, v):
        counts = np.bincount((x * 256).astype(np.int64), minlength=256)
        chi2 = stats.chisquare(counts).pvalue
        assert chi2 > 1e-4, chi2
        ks = stats.kstest(x[:10**6], "uniform").pvalue
        assert ks > 1e-4, ks
    joint = np.bincount((u * 16).astype(np.int64) * 16 + (v * 16).astype(np.int64),
                        minlength=256)
    assert stats.chisquare(joint).pvalue > 1e-4
    # different steps give different streams
    u2, _ = oracle.uniforms(20261202, r[:1000], j[:1000], 78)
    assert np.mean(u2 == u[:1000]) < 0.01
