"""Pins of the oracle's C twin (oracle/native.py, oracle/csrc/oracle_c.c) used by the
full-size GPU checks: the exact-operation fp32 k-means and the integer SIP sampler
must reproduce the pinned numpy forms (oracle/ibcs.py, oracle/sip.py) bit for bit,
and the same golden values and library cross-checks hold for them directly."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import kmeans_rounding_case as case
from oracle import native
from oracle.ibcs import kmeans_fp32
from oracle.sip import SIP_ONE, budget, sample_rows
from test_oracle_sip import _load_golden

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("N,d,qb,C,T,bf16", [(300, 64, 64, 4, 4, False), (1000, 128, 128, 8, 4, True),
                                             (777, 128, 128, 8, 1, True), (133, 64, 64, 16, 3, False),
                                             (200, 128, 128, 128, 2, True), (69, 64, 64, 8, 4, True)])
def test_kmeans_twin_equals_numpy_oracle(N, d, qb, C, T, bf16):
    rng = np.random.default_rng(N + d + C)
    base = rng.standard_normal((2, 1, N, d)).astype(np.float32)
    Q = (base + 0.5 * rng.standard_normal((2, 1, N, d))).astype(np.float32)
    if bf16:
        Q = _bf16(Q)
    mu, sz, a = native.kmeans_all(Q, qb, C, T)
    nqb = -(-N // qb)
    for b in range(2):
        for i in range(nqb):
            lo, hi = i * qb, min(N, (i + 1) * qb)
            rmu, rsz, ra = kmeans_fp32(Q[b, 0, lo:hi], C, T)
            assert np.array_equal(mu[b, 0, i].view(np.uint32), rmu.view(np.uint32)), (b, i)
            assert np.array_equal(sz[b, 0, i], rsz), (b, i)
            assert np.array_equal(a[b, 0, lo:hi], ra), (b, i)


@pytest.mark.parametrize("dim", [64, 128])
def test_kmeans_twin_takes_the_fused_assignment(dim):
    """The block where separately rounded multiplies and adds would flip one
    assignment (exact-rational construction): the twin takes the fused one."""
    X, row, fused, separate = case.build(dim)
    _, _, a = native.kmeans_all(X[None, None], X.shape[0], 2, 1)
    assert int(a[0, 0, row]) == fused != separate


@pytest.mark.parametrize("nkb,density", [(16, 0.25), (37, 0.3), (1024, 0.1), (2363, 0.08), (4725, 0.05),
                                         (300, 0.99), (50, 1.0), (7425, 0.08)])
def test_sampler_twin_equals_numpy_oracle(nkb, density):
    rng = np.random.default_rng(nkb)
    rows = 6
    logits = rng.standard_normal((1, 2, rows // 2, nkb)) * 2.0
    logits[rng.random(logits.shape) < 6.0 / nkb] += 12.0
    sc = np.exp(logits - logits.max(axis=-1, keepdims=True))
    sc = (sc / sc.sum(axis=-1, keepdims=True)).astype(np.float32)
    sc[0, 0, 0, :3] = [0.0, -1.0, np.nan]
    sc[0, 1, 0, 0] = 2.0
    sc[0, 0, 1, 1 % nkb] = 2.0 ** -30
    seed = 0x1234_5678_9ABC + nkb
    got = native.sample_all(sc, density, seed, with_thresholds=True)
    keys = [(0, h, i) for h in range(2) for i in range(rows // 2)]
    ref = sample_rows(sc, density, seed, keys)
    for (b, h, i), o in ref.items():
        c = int(got["counts"][b, h, i])
        assert c == o["count"], (b, h, i)
        assert np.array_equal(got["idx"][b, h, i, :c], o["idx"])
        assert np.array_equal(got["weight"][b, h, i, :c].view(np.uint32), o["weight"].view(np.uint32))
        assert np.array_equal(got["mask"][b, h, i], o["mask"])
        assert np.array_equal(got["thresh"][b, h, i], o["thresh"])


def test_sampler_twin_golden_waterfill():
    for g in _load_golden("sip_waterfill.txt"):
        s = np.array(g["scores"], dtype=np.float32)[None, None, None]
        assert native.budget(g["density"][0], s.shape[-1]) == g["budget"][0]
        got = native.sample_all(s, g["density"][0], 0, with_thresholds=True)
        assert got["thresh"][0, 0, 0].tolist() == g["thresholds"]


def test_budget_twin():
    for rho, nkb in [(1.0, 16), (0.25, 16), (0.10, 1024), (0.08, 2363), (0.08, 7425), (1e-9, 100), (0.5, 3),
                     (0.3, 37), (0.05, 4725)]:
        assert native.budget(rho, nkb) == budget(rho, nkb)


def test_philox_twin_matches_rocrand():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("g++ or rocRAND headers not available")
    exe = os.path.join(HERE, "..", "_build", "philox_rocrand_check_native")
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    subprocess.run([gxx, "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(HERE, "philox_rocrand_check.cpp"), "-o", exe], check=True)
    rng = np.random.default_rng(99)
    seeds = [int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)) for _ in range(200)] + [0, 2**64 - 1]
    ctr = rng.integers(0, 2**32, size=(len(seeds), 4), dtype=np.uint64).astype(np.uint32)
    ctr[:, 1] &= 0x3FFFFFFF  # the checker passes 4 * (c0 + 2^32 c1) as rocRAND's 64-bit offset
    text = "".join(f"{s} {c[0]} {c[1]} {c[2]} {c[3]}\n" for s, c in zip(seeds, ctr))
    res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    ref = np.array([[int(t) for t in line.split()] for line in res.stdout.strip().splitlines()], dtype=np.uint64)
    key = np.array([[s & 0xFFFFFFFF, s >> 32] for s in seeds], dtype=np.uint32)
    got = native.philox4x32_10(ctr, key).astype(np.uint64)
    np.testing.assert_array_equal(got, ref)


def test_sampler_twin_keep_frequency():
    """P5 statistics on the twin directly: keep frequency of each block over seeds within
    a binomial 5-sigma band of t / 2^24."""
    rng = np.random.default_rng(5)
    raw = rng.lognormal(0.0, 2.0, size=(1, 1, 1, 64))
    s = (raw / raw.sum()).astype(np.float32)
    seeds = 2000
    keep = np.zeros(64)
    t = None
    for sd in range(seeds):
        o = native.sample_all(s, 0.2, sd, with_thresholds=True)
        bits = np.unpackbits(o["mask"].view(np.uint8), bitorder="little")[:64]
        keep += bits
        t = o["thresh"][0, 0, 0]
    p = t.astype(np.float64) / SIP_ONE
    sd_ = np.sqrt(p * (1 - p) / seeds)
    assert np.all(np.abs(keep / seeds - p) <= 5 * sd_ + 1e-12)
