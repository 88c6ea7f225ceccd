"""Host-side accounting of bench.py: the position launches of a verify call
without per-row outputs (the schedule the dspark_verify header documents) and
the number of target rows it reads, checked against what strict prefix
semantics fix: every row that can decide a request is read, no row past its
L_b + 1 is, and a request whose first rejection lies in positions 1-4 reads
nothing more."""
import random

import pytest

import bench


@pytest.mark.parametrize("K", list(range(0, 41)))
def test_position_launches_cover_every_position_once(K):
    launches = bench.verify_position_launches(K)
    assert launches[0] == (1, min(4, K + 1))
    covered = []
    for j0, j1 in launches:
        assert j0 <= j1
        covered += list(range(j0, j1 + 1))
    assert covered == list(range(1, K + 2))
    assert len(launches) <= 2


def test_rows_read_bounds_and_cases():
    rng = random.Random(7)
    for K in (0, 1, 3, 4, 8, 16):
        for _ in range(300):
            L = rng.randint(0, K)
            a = rng.randint(0, L)
            n = bench.target_rows_read([L], [a], K)
            # the deciding rows: 1 .. a + 1 (the first rejection, or the bonus
            # row L + 1 when every drafted token was accepted)
            assert min(a + 1, L + 1) <= n <= L + 1
            if a < min(4, L):
                # rejected inside the first launch: only that launch's rows
                assert n == min(4, L + 1)
            if a >= 4 or a == L:
                assert n == L + 1


def test_rows_read_sums_over_requests():
    L = [16, 16, 16, 3, 0]
    a = [0, 5, 16, 3, 0]
    per = [bench.target_rows_read([l], [x], 16) for l, x in zip(L, a)]
    assert per == [4, 17, 17, 4, 1]
    assert bench.target_rows_read(L, a, 16) == sum(per)


def test_stored_counters_follow_the_kernel_sources(monkeypatch):
    """The committed counter figures are reported only while the dominant
    kernel's sources hash to the value stored beside them; the vector-ALU view
    is built from them and is null without them."""
    text = open(bench.PMC_SUMMARY).read()
    stored_hash = [l.split(":", 1)[1].strip() for l in text.splitlines()
                   if l.startswith("source_hash:")][0]
    monkeypatch.setattr(bench, "dominant_source_hash", lambda: stored_hash)
    got = bench.stored_counters()
    assert got is not None
    assert got["traffic_bytes_per_launch"] > 0 and got["valu_instructions_per_launch"] > 0
    view = bench.alu_view(got, 60e-6)
    ops = 64 * (got["valu_instructions_per_launch"] + got["valu_trans_instructions_per_launch"])
    assert view["lane_ops_per_launch"] == ops
    assert abs(view["frac"] - ops / 60e-6 / 1e12 / bench.VALU_PEAK_TOPS) < 1e-3
    monkeypatch.setattr(bench, "dominant_source_hash", lambda: "0" * 16)
    assert bench.stored_counters() is None
    assert bench.alu_view(None, 60e-6) is None
