"""Pins for the oracle's Philox4x32-10 (CPU only).

* rocRAND's ``philox4x32_10`` engine, an installed library built here as a
  host program, must give the same block outputs for random keys and
  counters, including the all-zero and all-ones corners;
* the uniform mapping u = (x0 >> 8) * 2^-24 lies on the 2^-24 grid in
  [0, 1 - 2^-24] and passes a Kolmogorov-Smirnov test on 10^6 draws;
* draws for different purposes / positions / rows are different streams.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_block(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND host driver")
    exe = str(tmp_path_factory.mktemp("philox") / "rocrand_philox_host")
    src = os.path.join(HERE, "philox_pin", "rocrand_philox_host.cpp")
    subprocess.run([hipcc, "-O1", "-o", exe, src], check=True, capture_output=True, cwd="/tmp")

    def run(rows):
        text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_rocrand(rocrand_block):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2**32, size=(20000, 6), dtype=np.uint64)
    rows[0] = 0
    rows[1] = 2**32 - 1
    rows[2, :2] = 0
    rows[3, 2:] = 0
    ref = rocrand_block(rows)
    got = np.stack(philox.philox4x32_10(rows[:, 2:].T, rows[:, :2].T), axis=1)
    assert np.array_equal(got, ref)


def test_verify_keying_matches_rocrand(rocrand_block):
    """The (seed, b, i, purpose, step) keying is the block at counter
    (b, i, purpose, step) under key (seed lo, seed hi)."""
    seed = 0x0123456789ABCDEF
    b, i = np.meshgrid(np.arange(300), np.arange(9), indexing="ij")
    b, i = b.ravel(), i.ravel()
    rows = np.stack([np.full_like(b, seed & 0xFFFFFFFF), np.full_like(b, seed >> 32),
                     b, i, np.full_like(b, philox.PURPOSE_RESIDUAL), np.full_like(b, 77)],
                    axis=1).astype(np.uint64)
    ref = rocrand_block(rows)
    u = philox.uniform(seed, b, i, philox.PURPOSE_RESIDUAL, 77)
    assert np.array_equal(u, (ref[:, 0] >> np.uint64(8)).astype(np.float64) * 2.0**-24)


def test_uniform_grid_and_range():
    u = philox.uniform(99, np.arange(1 << 16), 3, philox.PURPOSE_ACCEPT, 0)
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0**-24
    scaled = u * 2.0**24
    assert np.array_equal(scaled, np.floor(scaled))
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)   # exact in float32


def test_uniform_ks():
    b = np.arange(1_000_000)
    u = philox.uniform(2024, b % 1000, b // 1000, philox.PURPOSE_BONUS, 5)
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_streams_differ():
    b = np.arange(4096)
    a = philox.uniform(5, b, 0, philox.PURPOSE_ACCEPT, 0)
    r = philox.uniform(5, b, 0, philox.PURPOSE_RESIDUAL, 0)
    s = philox.uniform(5, b, 0, philox.PURPOSE_ACCEPT, 1)
    k = philox.uniform(6, b, 0, philox.PURPOSE_ACCEPT, 0)
    for other in (r, s, k):
        assert np.mean(a == other) < 0.01
        assert abs(np.corrcoef(a, other)[0, 1]) < 0.1
