"""Statistical evidence for the HIP path's draws at sizes the oracle cannot
enumerate, each law computed exactly (fp64) by the oracle from the same
rounded inputs:

* at V=1024, r=256, bf16 (the rank-256 MFMA draft strip and the MFMA residual
  strip, several vocabulary strips per row), 10^6 requests: the draft token at
  positions 1 and 2 follows p_d, the acceptance rate at position 1 is
  1 - TV(p_t, p_d) = sum_v min(p_t, p_d) (DSpark paper, section 3, the
  rejection-sampling verification), the next token after a rejection follows
  the normalised residual max(0, p_t - p_d), the bonus token follows the
  target row after the last accepted one, and the first emitted token follows
  p_t (the verification is lossless);
* the residual fallback (a rejection whose residual has no positive entry in
  floating point) draws from p_t and never the rejected token;
* acceptance outcomes are calibrated: P(accept x_k | prefix) equals
  alpha_k = sum_v min(p_t, p_d) within binomial error, and sequential
  temperature scaling (freeaitool DSpark guide, section 4.1) recovers a
  planted over-confidence from those labels.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsp():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import draft_sampling_verification_04_amd as d

    d.lib()
    return d


def chi2_p(counts, p, min_expect=20.0):
    """Chi-square p-value of counts against probabilities p; bins expected
    below min_expect are lumped into one."""
    counts = np.asarray(counts, np.float64)
    n = counts.sum()
    e = np.asarray(p, np.float64) * n
    big = e >= min_expect
    obs = np.append(counts[big], counts[~big].sum())
    exp = np.append(e[big], e[~big].sum())
    keep = exp > 0
    obs, exp = obs[keep], exp[keep]
    return float(stats.chi2.sf(((obs - exp) ** 2 / exp).sum(), len(obs) - 1))


def bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def test_rank256_multiblock_laws(dsp, orc):
    V, K, r, n, T, seed = 1024, 2, 256, 1_000_000, 0.8, 4242
    rng = np.random.default_rng(31)
    base_h = bf16_round(rng.normal(0, 1.5, (K, V)))
    A_h = bf16_round(rng.normal(0, 0.12, (V, r)))
    W_h = bf16_round(rng.normal(0, 0.12, (r, V)))
    rows_h = bf16_round(np.stack([base_h[0].float().numpy() + rng.normal(0, 1.0, V),
                                  base_h[1].float().numpy() + rng.normal(0, 1.0, V),
                                  rng.normal(0, 1.5, V)]))
    base32, A32, W32, rows32 = (t.float().numpy() for t in (base_h, A_h, W_h, rows_h))
    x0 = 3
    dev = "cuda"
    g_base = base_h.to(dev).expand(n, K, V).contiguous()
    g_A, g_W, g_rows = A_h.to(dev), W_h.to(dev), rows_h.to(dev)
    prev = torch.full((n,), x0, dtype=torch.int32, device=dev)
    temp = torch.full((n,), T, dtype=torch.float32, device=dev)
    tok, logp, lse = dsp.dspark_draft_sample(g_base, g_A, g_W, prev, temp, seed)
    offs = torch.zeros(n, dtype=torch.int64, device=dev)  # every request reads the same 3 rows
    acc, nxt, _, _ = dsp.dspark_verify(tok, prev, logp, lse, g_base, g_A, g_W, g_rows, offs, temp,
                                       seed, row_outputs=False)
    zero_len = torch.zeros(n, dtype=torch.int32, device=dev)
    acc0, nxt0, _, _ = dsp.dspark_verify(tok, prev, logp, lse, g_base, g_A, g_W, g_rows, offs,
                                         temp, seed + 1, zero_len, row_outputs=False)
    torch.cuda.synchronize()
    tok_c, acc_c, nxt_c = tok.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()
    assert (acc0.cpu().numpy() == 0).all()
    del g_base
    torch.cuda.empty_cache()

    # bit-exact against the oracle on the first requests
    m = 1000
    ob = np.broadcast_to(base32, (m, K, V))
    o_tok, _, _, o_gap = orc.draft_batch(ob, A32, W32, np.full(m, x0, np.int32),
                                         np.full(m, T, np.float32), seed)
    orv = orc.verify_batch(o_tok, np.full(m, x0, np.int32), ob, A32, W32, rows32,
                           np.zeros(m, np.int64), None, np.full(m, T, np.float32), seed)
    near = 0
    for b in range(m):
        if (tok_c[b] != o_tok[b]).any():
            assert o_gap[b].min() < P.NEAR_TIE, b
            near += 1
        elif acc_c[b] != orv["accepted"][b] or nxt_c[b] != orv["next_token"][b]:
            assert min(orv["accept_gap"][b], orv["next_gap"][b]) < P.NEAR_TIE, b
            near += 1
    assert near <= 2

    pd1 = orc.draft_probs(base32[0], A32, W32, x0, T)
    pt = [orc.target_probs(rows32[j], T) for j in range(3)]
    # draft position 1 and the marginal of position 2 (prev = x_1 varies)
    assert chi2_p(np.bincount(tok_c[:, 0], minlength=V), pd1) > 1e-4
    pd2 = np.stack([orc.draft_probs(base32[1], A32, W32, a, T) for a in range(V)])
    assert chi2_p(np.bincount(tok_c[:, 1], minlength=V), pd1 @ pd2) > 1e-4
    # acceptance rate at position 1 = sum min(p_t, p_d)
    alpha = np.minimum(pt[0], pd1).sum()
    rate = (acc_c >= 1).mean()
    assert abs(rate - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / n), (rate, alpha)
    # residual draw after a rejection at position 1
    rej = acc_c == 0
    res = np.maximum(pt[0] - pd1, 0.0)
    assert chi2_p(np.bincount(nxt_c[rej], minlength=V), res / res.sum()) > 1e-4
    # bonus draw after full acceptance (row 3) and with zero lengths (row 1)
    full = acc_c == K
    assert full.sum() > 50_000
    assert chi2_p(np.bincount(nxt_c[full], minlength=V), pt[2]) > 1e-4
    assert chi2_p(np.bincount(nxt0.cpu().numpy(), minlength=V), pt[0]) > 1e-4
    # losslessness: the first emitted token follows p_t
    z1 = np.where(acc_c >= 1, tok_c[:, 0], nxt_c)
    assert chi2_p(np.bincount(z1, minlength=V), pt[0]) > 1e-4
    print(f"alpha={alpha:.4f} rate={rate:.4f} rejected={rej.sum()} full={full.sum()} near={near}")


def _fallback_case(V=40, seed=17):
    """Target row 1 equals the draft row except at the drafted token x (logit
    -200 in the draft, -201 in the target): x's mass is far below the
    resolution of either normaliser, so p_t(v) == p_d(v) for v != x in floating
    point, the residual has no positive entry, and the accept ratio is e^-1."""
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 1, (1, V)).astype(np.float32)
    x = 7
    base[0, x] = -200.0
    target = np.stack([base[0], rng.normal(0, 1, V).astype(np.float32)])
    target[0, x] = -201.0
    return base, target, x


@pytest.mark.parametrize("factors", ["none", "zero_f32_r16", "zero_bf16_r256"])
def test_residual_fallback_branch(dsp, orc, factors):
    V, n, T, seed = 40, 200_000, 1.0, 99
    base, target, x = _fallback_case(V)
    ldt = torch.bfloat16 if factors == "zero_bf16_r256" else torch.float32
    r = {"none": 1, "zero_f32_r16": 16, "zero_bf16_r256": 256}[factors]
    # both values are exact in bf16, so every path sees the same inputs
    base = torch.from_numpy(base).to(ldt).float().numpy()
    target = torch.from_numpy(target).to(ldt).float().numpy()
    A0 = np.zeros((V, r), np.float32)
    W0 = np.zeros((r, V), np.float32)
    dev = "cuda"
    g_base = torch.from_numpy(base).to(dev, ldt).expand(n, 1, V).contiguous()
    g_rows = torch.from_numpy(target).to(dev, ldt)
    if factors == "none":
        g_A = g_W = None
    else:
        g_A = torch.from_numpy(A0).to(dev, ldt)
        g_W = torch.from_numpy(W0).to(dev, ldt)
    # the draft side's log-normaliser and log p_d(x), as the draft call reports them
    _, _, o_lse, _ = orc.draft_request(base, A0, W0, 0, T, seed, 0)
    logp_x = np.float32(np.float64(base[0, x]) - np.float64(o_lse[0]))
    tok = torch.full((n, 1), x, dtype=torch.int32, device=dev)
    prev = torch.zeros(n, dtype=torch.int32, device=dev)
    logp = torch.full((n, 1), float(logp_x), dtype=torch.float32, device=dev)
    lse = torch.full((n, 1), float(o_lse[0]), dtype=torch.float32, device=dev)
    temp = torch.full((n,), T, dtype=torch.float32, device=dev)
    offs = torch.zeros(n, dtype=torch.int64, device=dev)
    acc, nxt, _, _ = dsp.dspark_verify(tok, prev, logp, lse, g_base, g_A, g_W, g_rows, offs, temp,
                                       seed, row_outputs=False)
    torch.cuda.synchronize()
    acc_c, nxt_c = acc.cpu().numpy(), nxt.cpu().numpy()
    rej = acc_c == 0
    p_rej = 1.0 - np.exp(-1.0)
    assert abs(rej.mean() - p_rej) < 5 * np.sqrt(p_rej * (1 - p_rej) / n)
    assert not (nxt_c[rej] == x).any()
    pt = [orc.target_probs(target[j], T) for j in range(2)]
    assert chi2_p(np.bincount(nxt_c[rej], minlength=V), pt[0]) > 1e-4
    assert chi2_p(np.bincount(nxt_c[~rej], minlength=V), pt[1]) > 1e-4
    # request by request against the oracle, which takes the fallback branch
    m = 2000
    orv = orc.verify_batch(np.full((m, 1), x, np.int32), np.zeros(m, np.int32),
                           np.broadcast_to(base, (m, 1, V)), A0, W0, target,
                           np.zeros(m, np.int64), None, np.full(m, T, np.float32), seed)
    o_rej = orv["accepted"] == 0
    assert (orv["branch"][o_rej] == orc.BRANCH_FALLBACK).all() and o_rej.any()
    mism = (acc_c[:m] != orv["accepted"]) | (nxt_c[:m] != orv["next_token"])
    ties = np.minimum(orv["accept_gap"], orv["next_gap"]) < P.NEAR_TIE
    assert not (mism & ~ties).any(), np.nonzero(mism & ~ties)[0][:5]
    assert (mism & ties).sum() <= 2


def test_acceptance_is_calibrated_and_sts_recovers_overconfidence(dsp):
    """Position k is labelled when x_1..x_{k-1} were accepted; its label is
    whether x_k was.  Over the labelled positions, sum(label - alpha) is within
    5 binomial standard deviations of zero at every position and in every
    alpha decile.  A confidence head over-confident by a factor 2 in logit
    space, sigmoid(2 logit(alpha)), is fitted back to per-position
    temperatures near 2 and its calibration error falls."""
    import bench
    from draft_sampling_verification_04_amd import inputs

    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=16384, K=4, V=4096, temps=(0.7, 1.0))
    dev = "cuda"
    inp = inputs.make_inputs(w, dev, seed=8)
    B, K, V = w.B, w.K, w.V
    it = (1.0 / inp["temp"]).view(B, 1)
    Wf = inp["W"].float()
    pt = [torch.softmax(inp["target"][:, k].float() * it, dim=-1) for k in range(K)]
    offs = inputs.dense_offsets(B, K, dev)
    alphas, labels, reached = [], [], []
    for s in range(4):
        tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                                 inp["temp"], 500 + s)
        prevs = torch.cat([inp["prev"].view(B, 1), tok[:, :-1]], dim=1).long()
        al = torch.empty((B, K), device=dev, dtype=torch.float64)
        for k in range(K):
            bias = inp["A"][prevs[:, k]].float() @ Wf
            pd = torch.softmax((inp["base"][:, k].float() + bias) * it, dim=-1)
            al[:, k] = torch.minimum(pd, pt[k]).double().sum(-1)
        acc, _, _, _ = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], inp["target"].reshape(-1, V), offs,
                                         inp["temp"], 600 + s, row_outputs=False)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()
        kk = np.arange(K)[None, :]
        alphas.append(al.clamp(1e-6, 1 - 1e-6).cpu().numpy())
        labels.append((kk < a[:, None]).astype(np.float64))
        reached.append(kk <= a[:, None])
    al, y, rc = (np.concatenate(x) for x in (alphas, labels, reached))
    for k in range(K):
        m = rc[:, k]
        dz = (y[m, k] - al[m, k]).sum() / np.sqrt((al[m, k] * (1 - al[m, k])).sum())
        assert abs(dz) < 5, (k, m.sum(), dz)
    av, yv = al[rc], y[rc]
    edges = np.quantile(av, np.linspace(0, 1, 11))
    for lo, hi in zip(edges[:-1], edges[1:]):
        m = (av >= lo) & (av <= hi)
        dz = (yv[m] - av[m]).sum() / np.sqrt((av[m] * (1 - av[m])).sum())
        assert abs(dz) < 5, (lo, hi, m.sum(), dz)
    # planted over-confidence, fitted on one half and measured on the other
    lg = np.log(al) - np.log1p(-al)
    craw = 1.0 / (1.0 + np.exp(-2.0 * lg))
    half = len(al) // 2
    taus = bench.sts_fit(craw[:half], y[:half], rc[:half])
    cc = bench.sts_apply(craw[half:], taus)
    re_ = rc[half:]
    e_raw = bench.ece(craw[half:][re_], y[half:][re_])
    e_sts = bench.ece(cc[re_], y[half:][re_])
    print("reached per position", rc.sum(0), "taus", np.round(taus, 3), "ece", e_raw, e_sts)
    for k in range(K):
        if rc[:half, k].sum() >= 3000:
            assert abs(taus[k] - 2.0) < 0.25, (k, taus)
    assert e_sts < 0.5 * e_raw
