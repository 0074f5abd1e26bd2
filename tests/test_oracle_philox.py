"""Pin: the oracle's Philox4x32-10 equals rocRAND's independent implementation.

rocRAND ships Philox4x32-10 as an open-source header; a small host program
calls it (tests/philox_rocrand_check.cpp) and the two streams must agree word
for word. Also checks elementary distribution properties of the 24-bit
uniforms the sampler uses.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.philox import philox4x32_10
from oracle.sip import uniforms24

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("g++ or rocRAND headers not available")
    out = tmp_path_factory.mktemp("philox") / "philox_rocrand_check"
    subprocess.run(
        [gxx, "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "philox_rocrand_check.cpp"), "-o", str(out)],
        check=True,
    )
    return str(out)


def test_philox_matches_rocrand(rocrand_exe):
    rng = np.random.default_rng(1234)
    cases = [(0, (0, 0, 0, 0)), (2**64 - 1, (0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF))]
    for _ in range(300):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = (int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)), int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32)))
        cases.append((seed, c))
    # counters the sampler actually uses: (j/4, i, h, b)
    for seed in (0, 1, 42):
        for g in range(8):
            cases.append((seed, (g, 3, 2, 0)))
    text = "".join(f"{s} {c[0]} {c[1]} {c[2]} {c[3]}\n" for s, c in cases)
    res = subprocess.run([rocrand_exe], input=text, capture_output=True, text=True, check=True)
    ref = np.array([[int(t) for t in line.split()] for line in res.stdout.strip().splitlines()], dtype=np.uint64)
    ctr = np.array([c for _, c in cases], dtype=np.uint32)
    key = np.array([[s & 0xFFFFFFFF, s >> 32] for s, _ in cases], dtype=np.uint32)
    got = philox4x32_10(ctr, key).astype(np.uint64)
    assert ref.shape == got.shape
    np.testing.assert_array_equal(got, ref)


def test_uniforms24_distribution():
    u = np.concatenate([uniforms24(seed, 0, 1, 2, 4096) for seed in range(16)]).astype(np.float64)
    assert u.max() < 2**24 and u.min() >= 0
    x = u / 2**24
    n = x.size
    # mean and variance of U(0,1) within 6 standard errors
    assert abs(x.mean() - 0.5) < 6 * np.sqrt(1 / 12 / n)
    assert abs(x.var() - 1 / 12) < 6 * np.sqrt(1 / 180 / n)
    # words of one counter are not identical across j mod 4
    a = uniforms24(7, 0, 0, 0, 8)
    assert len(set(a.tolist())) == 8


def test_uniforms_depend_on_every_counter_word():
    base = uniforms24(5, 0, 0, 0, 16)
    for args in [(6, 0, 0, 0), (5, 1, 0, 0), (5, 0, 1, 0), (5, 0, 0, 1)]:
        assert not np.array_equal(base, uniforms24(*args, 16))
