"""Pins of the oracle's random draws: Philox4x32-10, the Box-Muller
Gaussians of the projection matrix, and the sample positions.

Philox is pinned to an independent library implementation (rocRAND's host
Philox4x32-10, compiled here from its public header); the fp64 ln, sin/cos
and sqrt steps to libm; the Gaussian matrix to a normality test and to the
Box-Muller identities; the sample positions to closed forms and a
uniformity test.
"""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import gauss, hyperattn, philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("hipcc")
    inc = "/opt/rocm/include"
    if cxx is None or not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND header or host compiler missing")
    exe = str(tmp_path_factory.mktemp("pin") / "rocrand_philox")
    subprocess.check_call([cxx, "-O1", "-I" + inc, "-D__HIP_PLATFORM_AMD__",
                           os.path.join(HERE, "pins", "rocrand_philox.cpp"), "-o", exe])

    def run(queries):
        text = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in queries)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(12345)
    # rocRAND reaches counter word 1 through a 64-bit offset counted in
    # 32-bit words, so word 1 stays below 2^30 here.
    queries = [(0, 0, 0, 0, 0), (0, 1, 0, 0, 0), (1, 0, 0, 0, 0),
               (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1)]
    for _ in range(3000):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(x) for x in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        c[1] %= 2**30
        queries.append((seed, *c))
    ref = rocrand_philox(queries)
    for qi, (seed, c0, c1, c2, c3) in enumerate(queries):
        got = philox.philox4x32_10(c0, c1, c2, c3, seed & 0xFFFFFFFF, seed >> 32)
        assert [int(g) for g in got] == [int(x) for x in ref[qi]], (seed, c0, c1, c2, c3)


def test_philox_streams_match_rocrand(rocrand_philox):
    # The two streams the method draws: projections (j, 0, 0, 0) and
    # samples (j, node, head, 2*batch + 1).
    seed = 0x1234_5678_9ABC_DEF0
    w = philox.philox_words(seed, 64)
    ref = rocrand_philox([(seed, j, 0, 0, 0) for j in range(16)]).reshape(-1)
    assert np.array_equal(w, ref)
    w = philox.philox_words(seed, 40, c1=13, c2=7, c3=5)
    ref = rocrand_philox([(seed, j, 13, 7, 5) for j in range(10)]).reshape(-1)
    assert np.array_equal(w, ref)


def _ulps(a, b):
    return abs(a - b) / math.ulp(max(abs(b), 1e-300))


def test_neg2_log_u_vs_libm():
    rng = np.random.default_rng(1)
    xs = [0, 1, 2, 3, 2**31 - 1, 2**31, 2**32 - 2, 2**32 - 1] + [int(x) for x in rng.integers(0, 2**32, 20000)]
    worst = 0.0
    for x in xs:
        u = (x + 0.5) / 2.0**32
        ref = -2.0 * math.log(u)
        got = gauss.neg2_log_u(x)
        worst = max(worst, abs(got - ref) / max(abs(ref), 1e-300))
    assert worst < 1e-14, worst


def test_sincos_vs_libm():
    rng = np.random.default_rng(2)
    xs = [0, 1, 2**30 - 1, 2**30, 2**31 - 1, 2**31, 3 * 2**30, 2**32 - 1] + [int(x) for x in rng.integers(0, 2**32, 20000)]
    worst = 0.0
    for x in xs:
        th = 2.0 * math.pi * ((x + 0.5) / 2.0**32)
        c, s = gauss.sincos_2pi(x)
        worst = max(worst, abs(c - math.cos(th)), abs(s - math.sin(th)))
    assert worst < 4e-15, worst


def test_sqrt_newton_vs_libm():
    rng = np.random.default_rng(3)
    vals = [4.65e-10, 1e-9, 0.25, 0.5, 1.0, 2.0, 3.999999, 44.36, 1e6] + list(rng.uniform(0, 45, 20000))
    for v in vals:
        assert _ulps(gauss.sqrt_newton(v), math.sqrt(v)) <= 1.0, v


def test_box_muller_identities():
    rng = np.random.default_rng(4)
    for _ in range(2000):
        wa, wb = (int(x) for x in rng.integers(0, 2**32, 2))
        z0, z1 = gauss.box_muller(wa, wb)
        ua = (wa + 0.5) / 2.0**32
        ub = (wb + 0.5) / 2.0**32
        assert abs((z0 * z0 + z1 * z1) - (-2.0 * math.log(ua))) <= 1e-13 * max(1.0, -2.0 * math.log(ua))
        ang = math.atan2(z1, z0) % (2.0 * math.pi)
        d = abs(ang - 2.0 * math.pi * ub)
        assert min(d, 2.0 * math.pi - d) < 1e-12


def test_projections_are_standard_normal():
    z = np.concatenate([gauss.projections(seed, 128, 16).reshape(-1) for seed in range(40)])
    assert z.dtype == np.float32 and z.size == 40 * 2048
    assert abs(z.mean()) < 0.02 and abs(z.var() - 1.0) < 0.03
    assert stats.kstest(z.astype(np.float64), "norm").pvalue > 1e-3


def test_projections_shape_and_determinism():
    a = gauss.projections(7, 64, 7)
    b = gauss.projections(7, 64, 7)
    c = gauss.projections(8, 64, 7)
    assert a.shape == (7, 64) and a.dtype == np.float32
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # r*d elements are a prefix of the same stream: fewer bits = first rows
    assert np.array_equal(gauss.projections(7, 64, 3), a[:3])


def test_sample_positions_power_of_two_closed_form():
    # ns = 2^k: floor(w * 2^k / 2^32) is the top k bits of the word
    seed, b, h, node = 99, 1, 5, 3
    for k in (0, 1, 8, 17, 19):
        s = hyperattn.sample_positions(seed, b, h, node, 2**k, 333)
        w = philox.philox_words(seed, 333, c1=node, c2=h, c3=2 * b + 1)
        assert np.array_equal(s, (w >> np.uint64(32 - k)).astype(np.int64))


def test_sample_positions_uniform_and_distinct_streams():
    ns, m = 10, 200000
    s = hyperattn.sample_positions(0, 0, 0, 1, ns, m)
    assert s.min() >= 0 and s.max() < ns
    counts = np.bincount(s, minlength=ns)
    assert stats.chisquare(counts).pvalue > 1e-3
    base = hyperattn.sample_positions(0, 0, 0, 1, 1 << 20, 64)
    for other in [(0, 0, 0, 2), (0, 0, 1, 1), (0, 1, 0, 1), (1, 0, 0, 1)]:
        seed, b, h, node = other
        assert not np.array_equal(base, hyperattn.sample_positions(seed, b, h, node, 1 << 20, 64))
    # samples never reuse the projection stream (its last counter word is 0)
    assert hyperattn.sample_positions(5, 0, 0, 0, 2**32 - 1, 4).tolist() != \
        [int(w * (2**32 - 1)) >> 32 for w in philox.philox_words(5, 4)]
    assert len(hyperattn.sample_positions(0, 0, 0, 1, 100, 0)) == 0
