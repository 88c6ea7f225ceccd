"""Pins for the oracle's confidence-scheduled prefix selection (freeaitool
DSpark guide, sections 4.1-4.2: c_k is the conditional acceptance probability
and lengths come from a greedy sort with early stop against a profiled
throughput curve; yage.ai analysis, scheduler paragraph: stop before the
curve's knee; legalagi.cn reading, section 5: greedy solution of the global
throughput maximisation).

* Brute force over every allocation L in [0, K]^B for B, K <= 4: the greedy
  objective equals the best achievable (budget only, and with a curve whose
  knee lies below the budget, where the early stop binds).
* Survival products equal numpy's sequential fp32 cumulative product.
* Invariants: budget respected, lengths <= K, offsets are the scan of L + 1,
  monotone in the budget; tie-break (S desc, k asc, b asc); zero confidence.
"""
import itertools

import numpy as np
import pytest


def _objective(orc, S, L, B, curve):
    E = B + sum(S[b, :L[b]].astype(np.float64).sum() for b in range(B))
    N = B + int(np.sum(L))
    tau = 1.0 if curve is None else orc.curve_tau(curve[0], curve[1], N)
    return E / tau


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small(orc, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    K = int(rng.integers(1, 5))
    conf = rng.beta(4, 2, (B, K)).astype(np.float32)
    if seed % 4 == 0:
        conf[0, -1] = 0.0
    budget = int(rng.integers(B, B * (K + 1) + 2))
    knee = B + max(1, (budget - B) // 2)
    curves = [None,
              (np.array([0.0, budget]), np.array([1.0, 1.0])),            # flat to the budget
              (np.array([knee, 2.0 * knee]), np.array([1.0, 2.5]))]       # knee below budget
    for curve in curves:
        if curve is None:
            L, offs, S, n = orc.schedule(conf, budget)
        else:
            L, offs, S, n = orc.schedule(conf, budget, curve[0], curve[1])
        assert int(np.sum(L + 1)) <= max(budget, B)
        assert n == int(L.sum())
        best = -np.inf
        for alloc in itertools.product(range(K + 1), repeat=B):
            alloc = np.array(alloc)
            if np.sum(alloc + 1) > max(budget, B):
                continue
            best = max(best, _objective(orc, S, alloc, B, curve))
        assert _objective(orc, S, L, B, curve) >= best - 1e-12


def test_knee_below_budget_stops_early(orc):
    B, K = 4, 8
    conf = np.full((B, K), 0.5, np.float32)
    budget = B * (K + 1)
    no_curve, _, _, n0 = orc.schedule(conf, budget)
    assert n0 == B * K
    # latency doubles per extra token past N = B + 4: only high-survival items pay
    L, _, S, n = orc.schedule(conf, budget, np.array([B + 4.0, B + 5.0]), np.array([1.0, 1.5]))
    assert 4 <= n < B * K
    # every taken item has survival at least that of every untaken one
    taken = np.zeros((B, K), bool)
    for b in range(B):
        taken[b, :L[b]] = True
    assert S[taken].min() >= S[~taken].max()


def test_survival_is_sequential_fp32_product(orc):
    rng = np.random.default_rng(0)
    conf = rng.uniform(0, 1, (50, 16)).astype(np.float32)
    _, _, S, _ = orc.schedule(conf, 10**6)
    np.testing.assert_array_equal(S, np.cumprod(conf, axis=1, dtype=np.float32))


def test_invariants_and_monotone_budget(orc):
    rng = np.random.default_rng(1)
    B, K = 40, 16
    conf = rng.beta(8, 2, (B, K)).astype(np.float32)
    prev = None
    for budget in (0, B - 1, B, B + 1, 100, 300, 600, B * (K + 1), 10**6):
        L, offs, S, n = orc.schedule(conf, budget)
        assert (L >= 0).all() and (L <= K).all()
        assert offs[0] == 0 and (np.diff(offs) == L + 1).all()
        assert int(np.sum(L + 1)) <= max(budget, B)
        assert n == min(max(budget - B, 0), B * K)
        if prev is not None:
            assert (L >= prev).all()
        prev = L


def test_tie_break_k_then_b(orc):
    conf = np.ones((3, 4), np.float32)
    L, _, _, n = orc.schedule(conf, 3 + 5)
    assert n == 5
    np.testing.assert_array_equal(L, [2, 2, 1])


def test_zero_confidence_is_never_selected(orc):
    conf = np.full((3, 5), 0.9, np.float32)
    conf[1, 2] = 0.0
    L, _, S, _ = orc.schedule(conf, 100)
    np.testing.assert_array_equal(L, [5, 2, 5])
    assert S[1, 2:].max() == 0.0


def test_curve_tau_piecewise_linear(orc):
    cn, ct = np.array([4.0, 8.0, 12.0]), np.array([1.0, 1.0, 3.0])
    assert orc.curve_tau(cn, ct, 0.0) == 1.0
    assert orc.curve_tau(cn, ct, 6.0) == 1.0
    assert orc.curve_tau(cn, ct, 10.0) == 2.0
    assert orc.curve_tau(cn, ct, 16.0) == 5.0  # extended with the last slope
