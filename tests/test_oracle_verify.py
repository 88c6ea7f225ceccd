"""Pins for the oracle's verification (yage.ai DSpark analysis, paragraphs on
prefix matching and on rejection sampling needing the exact draft probability;
legalagi.cn reading, section 3: the kept prefix is the longest accepted one and
the output distribution is the target's).

* Losslessness by exact enumeration (V <= 6, K <= 3): the emitted tokens,
  completed with target draws, have exactly the target's joint law.
* The oracle's Philox-driven sampler agrees with that law (chi-square over
  10^6 independent request streams), and its acceptance rate is 1 - TV.
* Special cases: T = 0 greedy rule, p_t == p_d (everything accepted),
  disjoint supports (always rejected, next ~ p_t), L = 0 (bonus only).
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp


class PrefixTargets:
    """Target logits as an arbitrary (seeded) function of the token prefix."""

    def __init__(self, V, seed, sd=1.5, shift=None):
        self.V, self.seed, self.sd, self.shift = V, seed, sd, shift
        self.cache = {}

    def __call__(self, prefix):
        prefix = tuple(int(x) for x in prefix)
        if prefix not in self.cache:
            h = self.seed
            for t in prefix:
                h = h * 1000003 + t + 1
            rng = np.random.default_rng(h % (2**63))
            row = rng.normal(0, self.sd, self.V)
            if self.shift is not None:
                row = row + self.shift
            self.cache[prefix] = row.astype(np.float32)
        return self.cache[prefix]


def _draft_problem(seed, V, K, r=3):
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 1.2, (K, V)).astype(np.float32)
    A = rng.normal(0, 0.8, (V, r)).astype(np.float32)
    W = rng.normal(0, 0.8, (r, V)).astype(np.float32)
    return base, A, W


@pytest.mark.parametrize("V,K,T", [(4, 2, 1.0), (5, 3, 0.7), (3, 3, 1.0), (6, 1, 1.3),
                                   (4, 3, 0.0), (5, 2, 0.0), (8, 3, 1.0), (8, 3, 0.6),
                                   (8, 3, 0.0)])
def test_lossless_by_exact_enumeration(orc, V, K, T):
    base, A, W = _draft_problem(10 * V + K, V, K)
    tgt = PrefixTargets(V, seed=V * 31 + K, shift=base[0] * 0.5)
    prev0 = 1
    got = orc.emitted_distribution(base, A, W, prev0, T, tgt)
    ref = orc.target_joint(tgt, T, V, K + 1)
    assert abs(sum(got.values()) - 1.0) < 1e-12
    for key in set(got) | set(ref):
        assert abs(got.get(key, 0.0) - ref.get(key, 0.0)) < 1e-12, key


def test_enumeration_catches_a_wrong_residual(orc, monkeypatch):
    """The enumeration pin is sharp: with the residual taken the wrong way round
    the emitted law is no longer the target's."""
    V, K, T = 4, 2, 1.0
    base, A, W = _draft_problem(77, V, K)
    tgt = PrefixTargets(V, seed=5)
    good = orc.emitted_distribution(base, A, W, 0, T, tgt)
    ref = orc.target_joint(tgt, T, V, K + 1)
    assert max(abs(good[k] - ref[k]) for k in ref) < 1e-12
    # plant the mistake in the oracle: residual taken as max(0, p_d - p_t)
    monkeypatch.setattr(orc, "_residual_mass", lambda pt, pd: np.maximum(pd - pt, 0.0))
    bad = orc.emitted_distribution(base, A, W, 0, T, tgt)
    assert max(abs(bad.get(k, 0.0) - ref[k]) for k in ref) > 1e-3


def _run_sampler(orc, base, A, W, prev0, T, tgt, n, seed, L=None):
    """Draft and verify n independent requests with the oracle's sampler.  The
    target rows of each request are built from that request's drafted prefix."""
    K, V = base.shape
    bases = np.ascontiguousarray(np.broadcast_to(base, (n, K, V)))
    tok, _, _, _ = orc.draft_batch(bases, A, W, np.full(n, prev0, np.int32),
                                   np.full(n, T, np.float32), seed)
    Lb = K if L is None else L
    rows = np.empty((n, Lb + 1, V), np.float32)
    for j in range(Lb + 1):
        keys = [tuple(t) for t in tok[:, :j]] if j else [()] * n
        uniq = {}
        for i, kk in enumerate(keys):
            uniq.setdefault(kk, []).append(i)
        for kk, idx in uniq.items():
            rows[idx, j] = tgt(kk)
    offs = np.arange(n, dtype=np.int64) * (Lb + 1)
    res = orc.verify_batch(tok, np.full(n, prev0, np.int32), bases, A, W,
                           rows.reshape(-1, V), offs,
                           None if L is None else np.full(n, L, np.int32),
                           np.full(n, T, np.float32), seed)
    return tok, res


def test_chi_square_first_two_emitted_tokens(orc):
    V, K, T, n = 8, 2, 1.0, 1_000_000
    base, A, W = _draft_problem(123, V, K)
    tgt = PrefixTargets(V, seed=321, sd=1.0, shift=base[0] * 0.7)
    tok, res = _run_sampler(orc, base, A, W, 3, T, tgt, n, seed=2024)
    acc, nxt = res["accepted"], res["next_token"]
    z1 = np.where(acc >= 1, tok[:, 0], nxt)
    z2 = np.where(acc >= 2, tok[:, 1], np.where(acc == 1, nxt, -1))
    # complete the second token with a target draw where only one was emitted
    rng = np.random.default_rng(9)
    need = np.nonzero(z2 < 0)[0]
    for a in range(V):
        idx = need[z1[need] == a]
        if len(idx):
            z2[idx] = rng.choice(V, size=len(idx), p=orc.target_probs(tgt((a,)), T))
    p1 = orc.target_probs(tgt(()), T)
    c1 = np.bincount(z1, minlength=V)
    chi = ((c1 - n * p1) ** 2 / (n * p1)).sum()
    assert stats.chi2.sf(chi, V - 1) > 1e-3
    joint = orc.target_joint(tgt, T, V, 2)
    expect = np.array([[joint[(a, b)] for b in range(V)] for a in range(V)]) * n
    counts = np.zeros((V, V))
    np.add.at(counts, (z1, z2), 1)
    chi = ((counts - expect) ** 2 / expect).sum()
    assert stats.chi2.sf(chi, V * V - 1) > 1e-3


def test_acceptance_rate_is_one_minus_tv(orc):
    V, K, T, n = 8, 1, 0.9, 200_000
    base, A, W = _draft_problem(7, V, K)
    tgt = PrefixTargets(V, seed=8, sd=1.3, shift=base[0])
    tok, res = _run_sampler(orc, base, A, W, 2, T, tgt, n, seed=77)
    pd = orc.draft_probs(base[0], A, W, 2, T)
    pt = orc.target_probs(tgt(()), T)
    p_acc = 1.0 - 0.5 * np.abs(pt - pd).sum()
    rate = (res["accepted"] >= 1).mean()
    assert abs(rate - p_acc) < 5 * np.sqrt(p_acc * (1 - p_acc) / n)
    # exact form in the enumeration: sum_v min(p_t, p_d)
    assert abs(np.minimum(pt, pd).sum() - p_acc) < 1e-12


def test_greedy_rule(orc):
    V, K = 9, 4
    base, A, W = _draft_problem(31, V, K)
    M = A.astype(np.float64) @ W.astype(np.float64)
    for trial in range(20):
        rng = np.random.default_rng(trial)
        tok, _, _, _ = orc.draft_request(base, A, W, 0, 0.0, 1, 0)
        target = rng.normal(0, 1, (K + 1, V)).astype(np.float32)
        # make a random number of leading positions agree with the draft
        agree = rng.integers(0, K + 1)
        for j in range(agree):
            target[j, tok[j]] = target[j].max() + 1.0
        res = orc.verify_request(tok, 0, base, A, W, target, K, 0.0, 1, 0)
        am = target.argmax(axis=1)
        a = 0
        while a < K and tok[a] == am[a]:
            a += 1
        assert res["accepted"] == a
        assert res["next_token"] == am[a]
    assert M.shape == (V, V)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_target_equal_to_draft_accepts_everything(orc, T):
    V, K, n = 7, 3, 3000
    base, A, W = _draft_problem(41, V, K)
    M = (A.astype(np.float64) @ W.astype(np.float64)).astype(np.float32)

    def tgt(prefix):  # the draft's own logits for the next position
        j = len(prefix)
        if j >= K:
            return base[K - 1]
        prev = 4 if j == 0 else prefix[-1]
        return base[j] + M[prev]

    # the oracle's bias is an fp64 sum rounded once, like M above
    _, res = _run_sampler(orc, base, A, W, 4, T, tgt, n, seed=5)
    assert (res["accepted"] == K).all()
    assert np.all(np.abs(res["row_logratio"].reshape(n, K + 1)[:, :K]) < 1e-6)


def test_disjoint_supports_always_reject(orc):
    V, K, n = 8, 2, 20000
    rng = np.random.default_rng(3)
    base = rng.normal(0, 1, (K, V)).astype(np.float32)
    base[:, 4:] = -1e4
    A = np.zeros((V, 2), np.float32)
    W = np.zeros((2, V), np.float32)
    trow = rng.normal(0, 1, V).astype(np.float32)
    trow[:4] = -1e4
    tgt = lambda prefix: trow
    tok, res = _run_sampler(orc, base, A, W, 0, 1.0, tgt, n, seed=12)
    assert (tok < 4).all()
    assert (res["accepted"] == 0).all()
    nxt = res["next_token"]
    assert (nxt >= 4).all()
    pt = orc.target_probs(trow, 1.0)[4:]
    c = np.bincount(nxt - 4, minlength=4)
    chi = ((c - n * pt) ** 2 / (n * pt)).sum()
    assert stats.chi2.sf(chi, 3) > 1e-3


def test_length_zero_gives_bonus_from_first_row(orc):
    V, K, n = 6, 3, 30000
    base, A, W = _draft_problem(9, V, K)
    trow = np.random.default_rng(4).normal(0, 1, V).astype(np.float32)
    tok, res = _run_sampler(orc, base, A, W, 1, 1.0, lambda p: trow, n, seed=3, L=0)
    assert (res["accepted"] == 0).all()
    pt = orc.target_probs(trow, 1.0)
    c = np.bincount(res["next_token"], minlength=V)
    chi = ((c - n * pt) ** 2 / (n * pt)).sum()
    assert stats.chi2.sf(chi, V - 1) > 1e-3


def test_row_outputs(orc):
    V, K = 50, 3
    base, A, W = _draft_problem(15, V, K)
    rng = np.random.default_rng(1)
    target = rng.normal(0, 2, (K + 1, V)).astype(np.float32)
    T = 0.7
    tok, _, _, _ = orc.draft_request(base, A, W, 0, T, 5, 2)
    res = orc.verify_request(tok, 0, base, A, W, target, K, T, 5, 2)
    it = np.float32(1.0) / np.float32(T)
    lse_ref = logsumexp((target * it).astype(np.float64), axis=1)
    np.testing.assert_allclose(res["row_lse_t"], lse_ref, rtol=1e-6)
    prev = 0
    for j in range(K):
        pd = orc.draft_probs(base[j], A, W, prev, T)
        pt = orc.target_probs(target[j], T)
        np.testing.assert_allclose(res["row_logratio"][j], np.log(pt[tok[j]]) - np.log(pd[tok[j]]),
                                   rtol=1e-5, atol=1e-5)
        prev = tok[j]
    assert res["row_logratio"][K] == 0.0


def _chi2_ok(counts, p, min_expect=20.0):
    """Chi-square of counts against probabilities p, with the bins expected
    below min_expect lumped into one."""
    n = counts.sum()
    e = p * n
    big = e >= min_expect
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(e[big], e[~big].sum())
    keep = exp > 0
    obs, exp = obs[keep], exp[keep]
    chi2 = ((obs - exp) ** 2 / exp).sum()
    return stats.chi2.sf(chi2, len(obs) - 1) > 1e-3


def _residual_case(seed_rng):
    V, r = 150, 4
    rng = np.random.default_rng(seed_rng)
    base = rng.normal(0, 1.0, (1, V)).astype(np.float32)
    A = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    W = rng.normal(0, 0.5, (r, V)).astype(np.float32)
    rows = np.stack([base[0] + rng.normal(0, 1.5, V), rng.normal(0, 1.2, V)]).astype(np.float32)
    return V, base, A, W, rows


def test_residual_draw_over_many_entries(orc):
    """After a rejection at position 1 the next token is the Gumbel-max over the
    positive entries of p_t - p_d (150 entries, 40k seeded draft-then-verify
    trials): it must follow normalise(max(0, p_t - p_d))."""
    V, base, A, W, rows = _residual_case(33)
    T, prev = 1.0, 3
    pd = orc.draft_probs(base[0], A, W, prev, T)
    pt = orc.target_probs(rows[0], T)
    res = np.maximum(pt - pd, 0.0)
    res /= res.sum()
    counts = np.zeros(V, np.int64)
    for seed in range(40000):
        tok, _, _, _ = orc.draft_request(base, A, W, prev, T, seed, 0)
        out = orc.verify_request(tok, prev, base, A, W, rows, 1, T, seed, 0)
        if out["accepted"] == 0:
            assert out["branch"] == orc.BRANCH_RESIDUAL
            counts[out["next_token"]] += 1
        else:
            assert out["branch"] == orc.BRANCH_BONUS
    assert counts.sum() > 10000
    assert _chi2_ok(counts, res)
    assert counts[res == 0].sum() == 0  # never an entry where p_t <= p_d


def test_bonus_draw_over_many_entries(orc):
    """With L = 0 the next token is the bonus draw from target row 1 (150
    entries, 30k trials); it must follow p_t."""
    V, base, A, W, rows = _residual_case(34)
    T, prev = 0.8, 5
    pt = orc.target_probs(rows[1], T)
    counts = np.zeros(V, np.int64)
    tok = np.zeros(1, np.int32)
    for seed in range(30000):
        out = orc.verify_request(tok, prev, base, A, W, rows[1:2], 0, T, seed, 0)
        assert out["branch"] == orc.BRANCH_BONUS
        counts[out["next_token"]] += 1
    assert _chi2_ok(counts, pt)


def fallback_case(V=40, seed=17):
    """A rejection whose residual p_t - p_d has no positive entry in fp64.

    Target row 1 equals the draft row except at the drafted token x, whose
    logit is -200 in the draft and -201 in the target: its mass (e^-200) is far
    below the fp64 resolution of either normaliser, so the two log-normalisers
    are bit-identical, p_t(v) == p_d(v) for every v != x, and p_t(x) < p_d(x).
    The accept ratio is exactly e^-1.  In exact arithmetic the residual law is
    p_t restricted to v != x, which is p_t to within e^-200: the fallback to
    p_t is the exact-arithmetic answer."""
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 1, (1, V)).astype(np.float32)
    x = 7
    base[0, x] = -200.0
    A = np.zeros((V, 2), np.float32)
    W = np.zeros((2, V), np.float32)
    target = np.stack([base[0], rng.normal(0, 1, V).astype(np.float32)])
    target[0, x] = -201.0
    return base, A, W, target, x


def test_residual_fallback_branch(orc):
    V = 40
    base, A, W, target, x = fallback_case(V)
    T, tok, N = 1.0, np.array([x], np.int32), 20000
    counts = np.zeros(V, np.int64)
    n_rej = 0
    for seed in range(N):
        out = orc.verify_request(tok, 0, base, A, W, target, 1, T, seed, 0)
        assert out["row_logratio"][0] == -1.0
        if out["accepted"] == 0:
            assert out["branch"] == orc.BRANCH_FALLBACK
            counts[out["next_token"]] += 1
            n_rej += 1
        else:
            assert out["branch"] == orc.BRANCH_BONUS
    p_rej = 1.0 - np.exp(-1.0)
    assert abs(n_rej / N - p_rej) < 5 * np.sqrt(p_rej * (1 - p_rej) / N)
    pt = orc.target_probs(target[0], T)
    assert counts[x] == 0
    assert _chi2_ok(counts, pt)
