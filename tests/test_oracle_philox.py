"""Pins for the oracle's counter-based RNG (Philox4x32-10, Salmon et al. SC'11).

* known-answer vectors of the published reference implementation (golden file);
* rocRAND's own Philox4x32-10 block function, run on the host, on random
  counters and keys;
* the uniform map is exact and inside (0, 1); uniforms pass a KS test;
* Gumbel draws have mean Euler-gamma and variance pi^2/6.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(x, 16) for x in line.split()])
    return rows


def test_philox_known_answers(orc):
    rows = _kat_rows()
    assert len(rows) == 3
    for w in rows:
        out = orc.philox4x32_10(w[:4], w[4:6])
        assert [int(x) for x in out] == w[6:]


def test_philox_matches_rocrand_host(orc, tmp_path):
    hipcc = shutil.which("hipcc")
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = tmp_path / "rr_ref"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O1", "-o", str(exe),
                           os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp")],
                          cwd=str(tmp_path))
    rng = np.random.default_rng(1234)
    words = rng.integers(0, 2**32, size=(200, 6), dtype=np.uint64)
    words[:10, 1:4] = 0  # small counters, as the sampler uses
    inp = "\n".join(" ".join("%x" % int(x) for x in row) for row in words) + "\n"
    res = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
    got = [[int(x, 16) for x in line.split()] for line in res.stdout.strip().splitlines()]
    assert len(got) == len(words)
    for row, ref in zip(words, got):
        out = orc.philox4x32_10(row[:4], row[4:6])
        assert [int(x) for x in out] == ref


def test_uniform_exact_and_open_interval(orc):
    # u = ((w >> 9) + 0.5) 2^-23 is exactly representable in fp32.
    for v in range(64):
        u = orc.uniform(7, 3, 2, 0, v)
        assert 0.0 < u < 1.0
        m = float(u) * 2**23 - 0.5
        assert m == int(m) and 0 <= m < 2**23
    # the word used for vocab index v is word v & 3 of the block at v >> 2
    key = [7 & 0xFFFFFFFF, 7 >> 32]
    for v in range(16):
        blk = orc.philox4x32_10([v >> 2, 2, 3, 0], key)
        w = int(blk[v & 3])
        assert float(orc.uniform(7, 3, 2, 0, v)) == ((w >> 9) + 0.5) * 2.0**-23


def test_uniform_ks_and_gumbel_moments(orc):
    n = 40000
    u = np.array([orc.uniform(11, b % 97, b // 97, 0, b % 1013) for b in range(n)], np.float64)
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    g = np.array([orc.gumbel(5, 1, 1, 0, v) for v in range(n)], np.float64)
    se_mean = np.sqrt(np.pi**2 / 6 / n)
    assert abs(g.mean() - np.euler_gamma) < 5 * se_mean
    assert abs(g.var() - np.pi**2 / 6) < 0.08
    # largest Gumbel the 23-bit uniform map can give
    umax = 1.0 - 2.0**-24
    assert g.max() <= -np.log(-np.log(umax)) + 1e-4
