"""Pins for the oracle's Markov-head draft (yage.ai DSpark analysis, paragraph on
the first-order Markov head; freeaitool DSpark guide, section 3.1).

Each test checks the oracle against something it does not share code with:
a closed form (one-hot factor rows reduce the rank-r lookup to a row of W),
a library routine (numpy matmul / scipy logsumexp), the W = 0 reduction to
independent per-position drafting, the T = 0 greedy rule, sampling
frequencies against exact probabilities, and the "of course / no problem"
toy that the pages use to motivate the head.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp


def _softmax64(z):
    z = np.asarray(z, np.float64)
    return np.exp(z - logsumexp(z))


def _rand_problem(seed, V=37, K=3, r=8, sd=0.6):
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 2.0, (K, V)).astype(np.float32)
    A = rng.normal(0, sd, (V, r)).astype(np.float32)
    W = rng.normal(0, sd, (r, V)).astype(np.float32)
    return base, A, W


@pytest.mark.parametrize("T", [1.0, 0.7, 1.9])
def test_one_hot_factor_rows_reduce_to_row_of_W(orc, T):
    base, _, W = _rand_problem(1)
    V, r = base.shape[1], W.shape[0]
    A = np.zeros((V, r), np.float32)
    A[np.arange(V), np.arange(V) % r] = 1.0  # row p of A selects row p mod r of W
    it = np.float32(1.0) / np.float32(T)
    for prev in (0, 5, 17, V - 1):
        p = orc.draft_probs(base[1], A, W, prev, T)
        s = base[1] + W[prev % r]  # fp32
        expect = _softmax64(s * it)
        np.testing.assert_allclose(p, expect, rtol=1e-12, atol=1e-15)
        assert abs(p.sum() - 1.0) < V * 2.0**-24


def test_dense_factor_matches_matrix_product(orc):
    base, A, W = _rand_problem(2, V=29, r=6)
    M = A.astype(np.float64) @ W.astype(np.float64)  # the full V x V transition matrix
    for prev in (0, 3, 28):
        s = base[0] + M[prev].astype(np.float32)
        np.testing.assert_allclose(orc.draft_probs(base[0], A, W, prev, 1.0), _softmax64(s),
                                   rtol=1e-6, atol=1e-12)
    # the bias follows the previous token: two prev tokens give different rows
    assert not np.allclose(orc.draft_probs(base[0], A, W, 0, 1.0),
                           orc.draft_probs(base[0], A, W, 3, 1.0))


def test_w_zero_is_independent_parallel_drafting(orc):
    base, A, _ = _rand_problem(3, V=1200, K=4)
    W = np.zeros((A.shape[1], base.shape[1]), np.float32)
    T, seed, b = 0.8, 99, 6
    it = np.float32(1.0) / np.float32(T)
    ref = None
    for prev0 in (0, 11, 52):
        tok, logp, lse, _ = orc.draft_request(base, A, W, prev0, T, seed, b)
        if ref is None:
            ref = tok
        np.testing.assert_array_equal(tok, ref)  # no dependence on the previous token
    # each position is a Gumbel-argmax of base_k / T with its own key
    for k in range(base.shape[0]):
        z = base[k] * it
        g = np.array([orc.gumbel(seed, b, k + 1, 0, v) for v in range(base.shape[1])], np.float32)
        assert ref[k] == int(np.argmax(z + g))
        np.testing.assert_allclose(lse[k], logsumexp(z.astype(np.float64)), rtol=1e-6)
        np.testing.assert_allclose(logp[k], z[ref[k]] - logsumexp(z.astype(np.float64)),
                                   rtol=1e-5, atol=1e-6)


def test_greedy_temperature_zero(orc):
    base, A, W = _rand_problem(4, V=61, K=5)
    M = A.astype(np.float64) @ W.astype(np.float64)
    tok, logp, lse, _ = orc.draft_request(base, A, W, 7, 0.0, 3, 0)
    prev = 7
    for k in range(base.shape[0]):
        s = base[k] + M[prev].astype(np.float32)
        assert tok[k] == int(np.argmax(s))
        assert logp[k] == 0.0
        np.testing.assert_allclose(lse[k], s.max(), rtol=1e-6)
        prev = tok[k]


def test_sampling_frequencies_match_markov_joint(orc):
    """Empirical joint of (x1, x2) over independent request streams equals
    p_d(x1 | x0) p_d(x2 | x1): the sampled token feeds the next step."""
    V, K, r = 6, 2, 3
    rng = np.random.default_rng(5)
    base = rng.normal(0, 1.0, (K, V)).astype(np.float32)
    A = rng.normal(0, 1.0, (V, r)).astype(np.float32)
    W = rng.normal(0, 1.0, (r, V)).astype(np.float32)
    T, prev0, n = 1.0, 2, 200000
    tok, _, _, _ = orc.draft_batch(np.broadcast_to(base, (n, K, V)), A, W,
                                   np.full(n, prev0, np.int32), np.full(n, T, np.float32), 17)
    counts = np.zeros((V, V))
    np.add.at(counts, (tok[:, 0], tok[:, 1]), 1)
    p1 = orc.draft_probs(base[0], A, W, prev0, T)
    expect = np.array([[p1[a] * orc.draft_probs(base[1], A, W, a, T)[c] for c in range(V)]
                       for a in range(V)]) * n
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert stats.chi2.sf(chi2, V * V - 1) > 1e-3


def test_of_course_no_problem_toy(orc):
    """Two continuations are each coherent ("of course", "no problem").  With no
    transition bias the positions are independent and half the drafts mix
    them; a pair bias in the rank-2 head drives that to ~0."""
    OF, COURSE, NO, PROBLEM = range(4)
    base = np.full((2, 4), -30.0, np.float32)
    base[0, [OF, NO]] = 0.0
    base[1, [COURSE, PROBLEM]] = 0.0
    A = np.zeros((4, 2), np.float32)
    A[OF] = [1, 0]
    A[NO] = [0, 1]

    def p_incoherent(W):
        p1 = orc.draft_probs(base[0], A, W, COURSE, 1.0)
        return (p1[OF] * orc.draft_probs(base[1], A, W, OF, 1.0)[PROBLEM]
                + p1[NO] * orc.draft_probs(base[1], A, W, NO, 1.0)[COURSE])

    W0 = np.zeros((2, 4), np.float32)
    assert abs(p_incoherent(W0) - 0.5) < 1e-12
    Wpair = np.zeros((2, 4), np.float32)
    Wpair[0, COURSE], Wpair[0, PROBLEM] = 6.0, -6.0
    Wpair[1, COURSE], Wpair[1, PROBLEM] = -6.0, 6.0
    exact = p_incoherent(Wpair)
    assert abs(exact - 1.0 / (1.0 + np.exp(12.0))) < 1e-12
    # and the sampler agrees
    n = 20000
    for W, want in ((W0, 0.5), (Wpair, exact)):
        tok, _, _, _ = orc.draft_batch(np.broadcast_to(base, (n, 2, 4)), A, W,
                                       np.full(n, COURSE, np.int32), np.ones(n, np.float32), 8)
        bad = np.mean(((tok[:, 0] == OF) & (tok[:, 1] == PROBLEM)) |
                      ((tok[:, 0] == NO) & (tok[:, 1] == COURSE)))
        assert abs(bad - want) < 5 * np.sqrt(max(want * (1 - want), 1e-4) / n)


def test_softmax_normalisation_and_lse(orc):
    base, A, W = _rand_problem(6, V=400, K=2, r=16)
    for T in (0.5, 1.0):
        p = orc.draft_probs(base[0], A, W, 9, T)
        assert abs(p.sum() - 1.0) < 400 * 2.0**-24
    tok, logp, lse, gap = orc.draft_request(base, A, W, 9, 1.0, 1, 2)
    p = orc.draft_probs(base[0], A, W, 9, 1.0)
    np.testing.assert_allclose(logp[0], np.log(p[tok[0]]), rtol=1e-5, atol=1e-6)
    assert (gap > 0).all()


def _draws(orc, base_k, A, W, prev, T, n, seed):
    """n independent single-position drafts (request index = stream)."""
    V = base_k.shape[0]
    tok, _, _, gap = orc.draft_batch(np.broadcast_to(base_k[None, None, :], (n, 1, V)), A, W,
                                     np.full(n, prev, np.int32), np.full(n, T, np.float32), seed)
    return tok[:, 0], gap[:, 0]


def _chi2_pvalue(counts, p, min_expect=20.0):
    """Chi-square p-value of counts against probabilities p, with the bins
    expected below min_expect lumped into one."""
    n = counts.sum()
    e = p * n
    big = e >= min_expect
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(e[big], e[~big].sum())
    keep = exp > 0
    obs, exp = obs[keep], exp[keep]
    return stats.chi2.sf(((obs - exp) ** 2 / exp).sum(), len(obs) - 1)


def test_draw_is_an_exact_softmax_sample_over_many_entries(orc):
    """Gumbel-max with one key per entry is an exact draw from softmax(z):
    100k independent request streams over 300 entries pass a chi-square test
    against the exact p_d.  The same statistic rejects a plausible mistake
    (the Gumbel's outer sign dropped: z + log(-log u), built from the oracle's
    own uniforms), so the test is sharp enough to see one."""
    V, r, n = 300, 4, 100_000
    rng = np.random.default_rng(21)
    base = rng.normal(0, 0.7, V).astype(np.float32)
    A = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W = rng.normal(0, 0.5, (r, V)).astype(np.float32)
    T, prev, seed = 0.9, 3, 5
    tok, _ = _draws(orc, base, A, W, prev, T, n, seed)
    p = orc.draft_probs(base, A, W, prev, T)
    assert (p * n >= 20).sum() > 250  # nearly every entry is its own bin
    assert _chi2_pvalue(np.bincount(tok, minlength=V), p) > 1e-3
    # the planted mistake, on 5000 streams: argmax z + log(-log u) instead of z + G
    it = np.float32(1.0) / np.float32(T)
    M = (A[prev].astype(np.float64) @ W.astype(np.float64)).astype(np.float32)
    z = (base + M) * it
    m = 5000
    wrong = np.empty(m, np.int64)
    for b in range(m):
        u = np.array([orc.uniform(seed, b, 1, 0, v) for v in range(V)], np.float64)
        wrong[b] = int(np.argmax(z + np.log(-np.log(u))))
    assert _chi2_pvalue(np.bincount(wrong, minlength=V), p) < 1e-6


def test_mass_in_one_range_draws_inside_it(orc):
    """Entries with no mass (logits -1e30) are never drawn; lse is that of the
    populated range (scipy)."""
    V, r = 300, 4
    rng = np.random.default_rng(8)
    base = np.full((3, V), -1e30, np.float32)
    lo, hi = 97, 181
    base[:, lo:hi] = rng.normal(0, 1.0, (3, hi - lo)).astype(np.float32)
    A = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W = np.zeros((r, V), np.float32)
    T, seed = 0.8, 13
    it = np.float32(1.0) / np.float32(T)
    for b in range(40):
        tok, logp, lse, _ = orc.draft_request(base, A, W, 0, T, seed, b)
        assert ((lo <= tok) & (tok < hi)).all()
    for k in range(3):
        z = base[k, lo:hi] * it
        np.testing.assert_allclose(lse[k], logsumexp(z.astype(np.float64)), rtol=1e-6)
