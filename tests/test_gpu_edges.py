"""GPU edge cases through the C ABI: exact ties (smallest index wins on every
path and across strips and lanes), the smallest batch and draft length,
extreme temperatures, a flat distribution, degenerate schedules,
verification with nothing drafted (K = 0), a one-entry vocabulary (V = 1), and
out-of-range token ids and lengths (clamped).  Where a
result has a closed form it is checked directly; elsewhere against the oracle
with the near-tie rule of tests/parity.py."""
import numpy as np
import pytest
import torch

import parity as P

pytestmark = pytest.mark.gpu

# (V, r, logit dtype, factor dtype): the rank-256 register-factor kernel, the
# runtime-rank MFMA kernel, the VALU path (fp32), and a vocabulary that is not a
# multiple of 8 (VALU path for bf16)
PATHS = [
    (2000, 256, torch.bfloat16, torch.bfloat16),
    (2000, 32, torch.bfloat16, torch.bfloat16),
    (2000, 16, torch.float32, torch.float32),
    (2003, 16, torch.bfloat16, torch.bfloat16),
]


@pytest.fixture(scope="module")
def dsp():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import draft_sampling_verification_04_amd as d

    d.lib()
    return d


def _zeros(B, K, V, r, ldt, fdt):
    dev = "cuda"
    return dict(base=torch.zeros((B, K, V), dtype=ldt, device=dev),
                A=torch.zeros((V, r), dtype=fdt, device=dev),
                W=torch.zeros((r, V), dtype=fdt, device=dev),
                prev=torch.arange(B, dtype=torch.int32, device=dev) % V,
                temp=torch.zeros(B, dtype=torch.float32, device=dev))


@pytest.mark.parametrize("V,r,ldt,fdt", PATHS)
def test_greedy_ties_take_the_smallest_index(dsp, V, r, ldt, fdt):
    B, K = 37, 3
    inp = _zeros(B, K, V, r, ldt, fdt)
    # every entry ties at 0: token 0 at every step
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 1)
    torch.cuda.synchronize()
    assert (tok == 0).all()
    assert (logp == 0).all() and (lse == 0).all()
    # two maxima, in different strips, lanes and (for 777 / 1500) MFMA tiles
    inp["base"][:, :, 1500] = 5.0
    inp["base"][:, :, 777] = 5.0
    inp["base"][:, 1, 3] = 5.0  # step 2: an earlier tie
    tok, _, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                          inp["temp"], 1)
    torch.cuda.synchronize()
    assert (tok[:, 0] == 777).all() and (tok[:, 1] == 3).all() and (tok[:, 2] == 777).all()
    assert torch.allclose(lse, torch.full_like(lse, 5.0))
    # verify at T = 0: accept iff the draft token is the target argmax (ties to
    # the smallest index); request 0's first row has its maximum at 5 and 9
    target = torch.zeros((B * (K + 1), V), dtype=ldt, device="cuda")
    target[:, 777] = 2.0
    target[1:, 3] = 2.0  # every row but request 0's first: tie between 3 and 777
    target[0, 5] = 3.0
    target[0, 9] = 3.0
    offs = torch.arange(B, dtype=torch.int64, device="cuda") * (K + 1)
    acc, nxt, rl, rr = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, offs, inp["temp"], 1)
    torch.cuda.synchronize()
    # request 0: row 1 argmax 5 != 777 -> reject at once, next = 5
    assert int(acc[0]) == 0 and int(nxt[0]) == 5
    # others: row 1 argmax is 3 (tie 3 / 777) != 777 -> reject at once, next = 3
    assert (acc[1:] == 0).all() and (nxt[1:] == 3).all()
    assert rr[0] == float("-inf")


@pytest.mark.parametrize("V,r,ldt,fdt", PATHS)
def test_single_request_single_step(dsp, orc, V, r, ldt, fdt):
    from draft_sampling_verification_04_amd import inputs

    w = inputs.resized(inputs.WORKLOADS["qwen3_4b"], B=1, K=1, V=V, r=r, dtype=ldt,
                       temps=(0.7,))
    inp = inputs.make_inputs(w, "cuda", seed=V + r)
    inp["A"] = inp["A"].to(fdt)
    inp["W"] = inp["W"].to(fdt)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 9)
    torch.cuda.synchronize()
    ora = P.oracle_draft(orc, inp, [0], 9)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), P.tol_for(ldt), tally)
    assert tally.compared + tally.near_ties == 1


@pytest.mark.parametrize("T", [0.05, 5.0])
def test_extreme_temperatures(dsp, orc, T):
    from draft_sampling_verification_04_amd import inputs

    w = inputs.resized(inputs.WORKLOADS["qwen3_4b"], B=40, K=3, V=3000, r=256, temps=(T,))
    inp = inputs.make_inputs(w, "cuda", seed=int(T * 100))
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 21)
    torch.cuda.synchronize()
    idx = [0, 7, 33, 39]
    ora = P.oracle_draft(orc, inp, idx, 21)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), P.tol_for(torch.bfloat16), tally)
    assert tally.compared >= 3 * len(idx) - 3
    # verify the same rows against the oracle
    V, K = w.V, w.K
    target = inp["target"].reshape(-1, V)
    for b in idx:
        tok[b] = torch.from_numpy(ora[b][0]).to(tok.device)
        logp[b] = torch.from_numpy(ora[b][1]).to(tok.device)
        lse[b] = torch.from_numpy(ora[b][2]).to(tok.device)
    offs = torch.arange(w.B, dtype=torch.int64, device="cuda") * (K + 1)
    acc, nxt, rl, rr = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, offs, inp["temp"], 21)
    torch.cuda.synchronize()
    rows = {b: P.np32(target[b * (K + 1):(b + 1) * (K + 1)]) for b in idx}
    orv = P.oracle_verify(orc, inp, idx, {b: ora[b][0] for b in idx}, rows, {b: K for b in idx},
                          21)
    P.compare_verify(acc.cpu().numpy(), nxt.cpu().numpy(), rl.cpu().numpy(), rr.cpu().numpy(),
                     offs.cpu().numpy(), orv, P.tol_for(torch.bfloat16), tally)
    print(tally)


def test_flat_distribution_is_decided_by_the_draws(dsp, orc):
    """Equal logits and no bias: every token is the Gumbel-argmax of the draws
    alone, so the GPU and the oracle must pick the same index."""
    B, K, V, r = 12, 4, 1024, 256
    inp = _zeros(B, K, V, r, torch.bfloat16, torch.bfloat16)
    inp["temp"].fill_(1.0)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 31)
    torch.cuda.synchronize()
    ora = P.oracle_draft(orc, inp, list(range(B)), 31)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), P.tol_for(torch.bfloat16), tally)
    assert tally.compared >= B * K - 2
    # lse of a flat row is log V, log p_d = -log V
    assert torch.allclose(lse, torch.full_like(lse, float(np.log(V))), rtol=1e-5)
    assert torch.allclose(logp, torch.full_like(logp, -float(np.log(V))), rtol=1e-5)


def test_degenerate_schedules(dsp):
    B, K = 50, 6
    conf = torch.rand((B, K), generator=torch.Generator().manual_seed(4)).to("cuda")
    # a budget that only covers the root tokens selects nothing
    L, offs, _ = dsp.dspark_schedule(conf, B)
    torch.cuda.synchronize()
    assert (L == 0).all()
    assert torch.equal(offs, torch.arange(B + 1, dtype=torch.int64, device="cuda"))
    L, offs, _ = dsp.dspark_schedule(conf, 3)  # budget below B
    torch.cuda.synchronize()
    assert (L == 0).all()
    # a budget past every item selects every position with S > 0
    conf[7, 2] = 0.0  # request 7 stops after its second position
    L, offs, surv = dsp.dspark_schedule(conf, 10 * B * K)
    torch.cuda.synchronize()
    expect = torch.full((B,), K, dtype=torch.int32, device="cuda")
    expect[7] = 2
    assert torch.equal(L, expect)
    assert int(offs[B]) == int((L + 1).sum())
    # a one-point curve is constant latency: the objective rises with every
    # positive item, so the result equals the plain budget rule
    L1, _, _ = dsp.dspark_schedule(conf, B + 40, [float(B + 40)], [1.0])
    L0, _, _ = dsp.dspark_schedule(conf, B + 40)
    torch.cuda.synchronize()
    assert torch.equal(L1, L0) and int(L0.sum()) == 40


@pytest.mark.parametrize("K", [1, 4])
def test_parallel_drafting_equals_zero_transition(dsp, orc, K):
    """No factors: every position is drawn from its own base logits.  The
    tokens equal the Markov path's with W = 0 (same draws, zero bias) on the
    GPU, and the oracle's with W = 0."""
    from draft_sampling_verification_04_amd import inputs

    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=70, K=K, V=3000, r=256)
    inp = inputs.make_inputs(w, "cuda", seed=40 + K, with_target=False)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], None, None, inp["prev"], inp["temp"], 17)
    Az = torch.zeros_like(inp["A"])
    Wz = torch.zeros_like(inp["W"])
    tz, lz, ez = dsp.dspark_draft_sample(inp["base"], Az, Wz, inp["prev"], inp["temp"], 17)
    torch.cuda.synchronize()
    assert torch.equal(tok, tz)
    # the two paths merge their partials in different orders, so lse_d may
    # differ in the last fp32 places (one ulp at |lse| ~ 20 is 1.9e-6)
    assert torch.allclose(lse, ez, rtol=0, atol=2e-5)
    assert torch.allclose(logp, lz, rtol=0, atol=2e-5)
    inp["A"], inp["W"] = Az, Wz
    idx = [0, 3, 31, 32, 69]
    ora = P.oracle_draft(orc, inp, idx, 17)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), P.tol_for(torch.bfloat16), tally)
    assert tally.compared >= len(idx) * K - 2
    # verify without factors (the zero-bias case, vector-ALU residual) equals
    # verify with zero factors (the rank-256 MFMA residual), and the oracle's
    # with W = 0
    g = torch.Generator(device="cuda").manual_seed(50 + K)
    target = (inp["base"][:, :1].float().expand(-1, K + 1, -1)
              + 1.5 * torch.randn((w.B, K + 1, w.V), generator=g, device="cuda"))
    target = target.to(torch.bfloat16).reshape(-1, w.V).contiguous()
    offs = inputs.dense_offsets(w.B, K, "cuda")
    a0, n0, r0, q0 = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], None, None,
                                       target, offs, inp["temp"], 23)
    a1, n1, r1, q1 = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], Az, Wz,
                                       target, offs, inp["temp"], 23)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1) and torch.equal(n0, n1)
    assert torch.equal(r0, r1) and torch.equal(q0, q1)
    assert int((a0 < K).sum()) > 10  # rejections: the residual draw ran
    rows = {b: P.np32(target[b * (K + 1):(b + 1) * (K + 1)]) for b in idx}
    orv = P.oracle_verify(orc, inp, idx, {b: tok[b].cpu().numpy() for b in idx}, rows,
                          {b: K for b in idx}, 23)
    P.compare_verify(a0.cpu().numpy(), n0.cpu().numpy(), r0.cpu().numpy(), q0.cpu().numpy(),
                     offs.cpu().numpy(), orv, P.tol_for(torch.bfloat16), tally)
    print(tally)
    assert tally.verify_clean >= len(idx) - 1


@pytest.mark.parametrize("V,ldt", [(3000, torch.bfloat16), (3001, torch.bfloat16),
                                   (3000, torch.float32)])
def test_verify_with_nothing_drafted(dsp, orc, V, ldt):
    """K = 0: no drafted token, so every request accepts none and its next token
    is the bonus draw from its single target row (row L_b + 1 = 1).  The draft
    inputs are empty and the factors absent (NULL at the boundary).  Greedy and
    sampled requests; whole 16-byte chunks (V = 3000) and a ragged row end
    (V = 3001); with and without the per-row outputs."""
    B, seed, dev = 70, 13, "cuda"
    g = torch.Generator().manual_seed(40 + V)
    target = (3.0 * torch.randn((B, V), generator=g)).to(ldt)
    temp = torch.tensor([(0.0, 0.7, 1.0)[b % 3] for b in range(B)], dtype=torch.float32)
    prev = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    no_tok = torch.empty((B, 0), dtype=torch.int32, device=dev)
    no_f = torch.empty((B, 0), dtype=torch.float32, device=dev)
    no_base = torch.empty((B, 0, V), dtype=ldt, device=dev)
    offs = torch.arange(B, dtype=torch.int64, device=dev)
    args = (no_tok, prev.to(dev), no_f, no_f, no_base, None, None, target.to(dev), offs,
            temp.to(dev), seed)
    acc, nxt, rl, _ = dsp.dspark_verify(*args)
    acc2, nxt2, _, _ = dsp.dspark_verify(*args, row_outputs=False)
    torch.cuda.synchronize()
    assert (acc == 0).all() and torch.equal(acc2, acc) and torch.equal(nxt2, nxt)
    t32 = P.np32(target)
    rl = rl.cpu().numpy()
    zA, zW = np.zeros((V, 1), np.float32), np.zeros((1, V), np.float32)
    near = 0
    for b in range(B):
        res = orc.verify_request(np.zeros(0, np.int32), int(prev[b]), np.zeros((0, V), np.float32),
                                 zA, zW, t32[b:b + 1], 0, float(temp[b]), seed, b)
        assert res["accepted"] == 0
        assert P.close(rl[b:b + 1], res["row_lse_t"], P.tol_for(ldt)), (b, rl[b], res["row_lse_t"])
        if int(nxt[b]) != res["next_token"]:
            assert res["next_gap"] < P.NEAR_TIE, (b, int(nxt[b]), res["next_token"])
            near += 1
    assert near <= 1


@pytest.mark.parametrize("ldt", [torch.float32, torch.bfloat16])
def test_one_entry_vocabulary(dsp, orc, ldt):
    """V = 1: draft and target put all mass on entry 0, so every drafted and
    every next token is 0, log p_d = 0 (up to the rounding of the key and its
    draw term) and every greedy draft is accepted.  A sampled draft is accepted
    unless log u >= -log p_d, which that rounding allows only for u within about
    1e-6 of 1.  Everything is also compared with the oracle."""
    B, K, V, r, seed, dev = 40, 3, 1, 16, 29, "cuda"
    g = torch.Generator().manual_seed(31)
    inp = dict(base=(2.0 * torch.randn((B, K, V), generator=g)).to(ldt).to(dev),
               A=(0.3 * torch.randn((V, r), generator=g)).to(ldt).to(dev),
               W=(0.3 * torch.randn((r, V), generator=g)).to(ldt).to(dev),
               prev=torch.zeros(B, dtype=torch.int32, device=dev),
               temp=torch.tensor([(0.0, 0.7, 1.0)[b % 3] for b in range(B)],
                                 dtype=torch.float32, device=dev))
    target = (2.0 * torch.randn((B * (K + 1), V), generator=g)).to(ldt).to(dev)
    offs = torch.arange(B, dtype=torch.int64, device=dev) * (K + 1)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], seed)
    acc, nxt, rl, rr = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, offs, inp["temp"], seed)
    torch.cuda.synchronize()
    assert (tok == 0).all() and (nxt == 0).all()
    greedy = inp["temp"] == 0
    assert (acc[greedy] == K).all() and int((acc[~greedy] != K).sum()) <= 1
    assert float(logp.abs().max()) < 1e-5
    idx = list(range(B))
    tol = P.tol_for(ldt)
    tally = P.Tally()
    ora = P.oracle_draft(orc, inp, idx, seed)
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), tol, tally)
    assert tally.draft_clean == B
    rows = {b: P.np32(target[b * (K + 1):(b + 1) * (K + 1)]) for b in idx}
    orv = P.oracle_verify(orc, inp, idx, {b: ora[b][0] for b in idx}, rows, {b: K for b in idx},
                          seed)
    P.compare_verify(acc.cpu().numpy(), nxt.cpu().numpy(), rl.cpu().numpy(), rr.cpu().numpy(),
                     offs.cpu().numpy(), orv, tol, tally)
    print(tally)
    assert tally.verify_clean >= B - 1


@pytest.mark.parametrize("V,r,dt", [(2056, 256, torch.bfloat16), (2003, 16, torch.float32)])
def test_out_of_range_ids_and_lengths_are_clamped(dsp, V, r, dt):
    """Token ids and lengths read from device memory are clamped before they
    index anything (ids to [0, V), lengths to [0, K]): out-of-range previous
    tokens, drafted tokens and lengths give exactly the results of their
    clamped values, on the rank-256 MFMA paths and on the fp32 VALU paths."""
    from draft_sampling_verification_04_amd import inputs as inputs_mod

    w = inputs_mod.resized(inputs_mod.WORKLOADS["long_draft"], B=24, K=4, V=V, r=r, dtype=dt)
    inp = inputs_mod.make_inputs(w, "cuda", seed=5)
    B, K = w.B, w.K
    bad_prev = inp["prev"].clone()
    bad_prev[0::4] = -7
    bad_prev[1::4] = V + 11
    args = (inp["base"], inp["A"], inp["W"])
    d_bad = dsp.dspark_draft_sample(*args, bad_prev, inp["temp"], 8)
    d_ok = dsp.dspark_draft_sample(*args, bad_prev.clamp(0, V - 1), inp["temp"], 8)
    torch.cuda.synchronize()
    for x, y in zip(d_bad, d_ok):
        assert torch.equal(x, y)
    tok, logp, lse = d_ok
    bad_tok = tok.clone()
    bad_tok[0::3, 0] = -3
    bad_tok[1::3, 1] = V + 5
    bad_len = torch.full((B,), K, dtype=torch.int32, device="cuda")
    bad_len[0::5] = -2
    bad_len[1::5] = K + 6
    bad_len[2::5] = 2
    target = inp["target"].reshape(-1, V)
    offs = inputs_mod.dense_offsets(B, K, "cuda")

    def verify(t, L, p):
        return dsp.dspark_verify(t, p, logp, lse, inp["base"], inp["A"], inp["W"], target, offs,
                                 inp["temp"], 8, L)

    v_bad = verify(bad_tok, bad_len, bad_prev)
    v_ok = verify(bad_tok.clamp(0, V - 1), bad_len.clamp(0, K), bad_prev.clamp(0, V - 1))
    torch.cuda.synchronize()
    for x, y in zip(v_bad, v_ok):
        assert torch.equal(x.nan_to_num(7.0), y.nan_to_num(7.0))
    assert int((v_ok[0] < bad_len.clamp(0, K)).sum()) >= 3  # some rejections (residual draws)
