"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes span several vocabulary strips and a ragged tail; the named workloads
run at their full sizes with the oracle on a sampled subset of requests
(requests are independent, so per-request parity at the real V, r and K is
complete evidence for those requests).  See tests/parity.py for the rules.
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

    d.lib()  # raises when the HIP library is missing
    return d


@pytest.fixture(scope="module")
def inputs():
    from draft_sampling_verification_04_amd import inputs as m

    return m


def _draft_and_verify(dsp, orc, inp, seed, idx, tol, lengths=None, row_off=None, target=None):
    """GPU draft on all requests, oracle on idx; then verify with the oracle's
    draft for idx (GPU draft elsewhere) and compare."""
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], seed)
    torch.cuda.synchronize()
    ora = P.oracle_draft(orc, inp, idx, seed)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), tol, tally)
    B, K, V = inp["base"].shape
    # verify inputs: oracle draft outputs on the sampled requests
    for b in idx:
        tok[b] = torch.from_numpy(ora[b][0]).to(tok.device)
        logp[b] = torch.from_numpy(ora[b][1]).to(tok.device)
        lse[b] = torch.from_numpy(ora[b][2]).to(tok.device)
    if target is None:
        target = inp["target"].reshape(-1, V)
        row_off = torch.arange(B, dtype=torch.int64, device=tok.device) * (K + 1)
    acc, nxt, rl, rr = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, row_off, inp["temp"], seed, lengths)
    # without per-row outputs only the rows that can decide the result are read
    # (positions 1-4, then 5..K+1 for requests with no rejection in 1-4)
    acc2, nxt2, rl2, rr2 = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                             inp["W"], target, row_off, inp["temp"], seed,
                                             lengths, row_outputs=False)
    torch.cuda.synchronize()
    assert rl2 is None and rr2 is None
    assert torch.equal(acc2, acc) and torch.equal(nxt2, nxt)
    L = {b: (K if lengths is None else int(lengths[b])) for b in idx}
    ro = row_off.cpu().numpy()
    rows = {b: P.np32(target[int(ro[b]):int(ro[b]) + L[b] + 1]) for b in idx}
    orv = P.oracle_verify(orc, inp, idx, {b: ora[b][0] for b in idx}, rows, L, seed)
    P.compare_verify(acc.cpu().numpy(), nxt.cpu().numpy(), rl.cpu().numpy(), rr.cpu().numpy(),
                     ro, orv, tol, tally)
    return tally, (tok, logp, lse, acc, nxt)


def test_tiny_full_parity(dsp, orc, inputs):
    w = inputs.WORKLOADS["tiny"]
    inp = inputs.make_inputs(w, "cuda", seed=0)
    tally, _ = _draft_and_verify(dsp, orc, inp, 0, list(range(w.B)), P.tol_for(w.dtype))
    print(tally)
    assert tally.near_ties <= 1
    assert tally.draft_clean >= w.B - 1 and tally.verify_clean >= w.B - 1


@pytest.mark.parametrize("V,r,K,B,ldt,fdt", [
    (3001, 32, 3, 6, torch.bfloat16, torch.bfloat16),
    (777, 16, 2, 3, torch.float32, torch.bfloat16),
    (5, 16, 4, 4, torch.bfloat16, torch.float32),
    (1, 16, 2, 2, torch.float32, torch.float32),
    (4099, 48, 5, 9, torch.float32, torch.float32),
    # rank 256 takes the register-factor kernel: a ragged last strip, a request
    # count that leaves lanes idle, and a one-chunk vocabulary
    (1000, 256, 3, 40, torch.bfloat16, torch.bfloat16),
    (8, 256, 2, 3, torch.bfloat16, torch.bfloat16),
    # four-wave groups (64 < B <= 128) and a last strip of 8 entries, so the
    # last draft block holds 8 entries
    (4104, 256, 3, 100, torch.bfloat16, torch.bfloat16),
    # the runtime-rank MFMA kernel with eight-wave groups (B > 128)
    (2056, 64, 2, 150, torch.bfloat16, torch.bfloat16),
])
def test_small_shapes_parity(dsp, orc, inputs, V, r, K, B, ldt, fdt):
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=B, K=K, V=V, r=r, dtype=ldt)
    inp = inputs.make_inputs(w, "cuda", seed=V + K)
    inp["A"] = inp["A"].to(fdt)
    inp["W"] = inp["W"].to(fdt)
    tally, _ = _draft_and_verify(dsp, orc, inp, 11, list(range(B)), P.tol_for(ldt))
    print(tally)
    # every request compared; at most one near-tie excused over the batch
    assert tally.near_ties <= 1
    assert tally.draft_clean >= B - 1 and tally.verify_clean >= B - 1


def _spread_requests(temp, n_min=16, extra=()):
    """At least n_min requests, the same number at every temperature present
    (spread over the batch), plus the first and last request."""
    t = temp.cpu().numpy()
    vals = sorted(set(t.tolist()))
    per = -(-n_min // len(vals))
    idx = [0, len(t) - 1]
    for v in vals:
        cand = np.nonzero(t == v)[0]
        pick = np.linspace(0, len(cand) - 1, min(per, len(cand))).round().astype(int)
        idx += [int(cand[i]) for i in pick]
    idx += [int(i) for i in extra if i < len(t)]
    return sorted(set(idx))


@pytest.mark.parametrize("name", ["qwen3_4b", "long_draft", "high_conc"])
def test_full_size_sampled_parity(dsp, orc, inputs, name):
    """Full-size workloads, every temperature: at least 16 requests compared
    with the oracle at the real V, r and K.  At most one near-tie divergence
    is expected over the sample, so every other request matches whole."""
    w = inputs.WORKLOADS[name]
    inp = inputs.make_inputs(w, "cuda", seed=1)
    idx = _spread_requests(inp["temp"], 16)
    tally, _ = _draft_and_verify(dsp, orc, inp, 5, idx, P.tol_for(w.dtype))
    temps = sorted(set(inp["temp"].cpu().numpy()[idx].tolist()))
    print(name, len(idx), temps, tally)
    assert len(idx) >= 16 and temps == sorted(set(np.float32(w.temps).tolist()))
    assert tally.near_ties <= 1
    assert tally.draft_clean >= len(idx) - 1 and tally.verify_clean >= len(idx) - 1
    del inp
    torch.cuda.empty_cache()


def test_misaligned_inputs(dsp, orc, inputs):
    """Logits and factors that start 2 bytes past a 16-byte boundary (views
    into a larger buffer) cannot take the kernels with 16-byte and direct-to-LDS
    loads; the library takes the element-load kernels instead (draft strip,
    verify rows and residual), with the same results against the oracle."""
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=24, K=3, V=2056)
    inp = inputs.make_inputs(w, "cuda", seed=4)

    def shifted(t):
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 == 2
        return v

    for k in ("base", "A", "W", "target"):
        inp[k] = shifted(inp[k])
    tally, (_, _, _, acc, _) = _draft_and_verify(dsp, orc, inp, 7, list(range(w.B)),
                                                 P.tol_for(w.dtype))
    print(tally)
    assert int((acc < w.K).sum()) >= 5  # rejections: the residual kernel ran
    assert tally.near_ties <= 1
    assert tally.draft_clean >= w.B - 1 and tally.verify_clean >= w.B - 1


def test_longest_draft_chain(dsp, orc, inputs):
    """A 64-step Markov chain (each token feeds the next step's factor row) on
    the rank-256 kernel, every request compared with the oracle, then verified
    over its 65 target rows (the second verify launch covers positions 5-65)."""
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=40, K=64, V=2056)
    inp = inputs.make_inputs(w, "cuda", seed=6)
    tally, (_, _, _, acc, _) = _draft_and_verify(dsp, orc, inp, 12, list(range(w.B)),
                                                 P.tol_for(w.dtype))
    print(tally, "accepted:", sorted(acc.cpu().numpy().tolist()))
    assert tally.near_ties <= 1
    assert tally.draft_clean >= w.B - 1 and tally.verify_clean >= w.B - 1
    assert tally.compared >= (w.B - 1) * w.K


@pytest.mark.parametrize("B", [4096, 4097])
def test_verify_tail_list_limits(dsp, orc, inputs, B):
    """The second verify launch lists in LDS the rows still needed by up to
    4096 requests: B = 4096 fills that list, and B = 4097 takes per-row launches
    instead.  Both equal verification with every row read, and the oracle on
    requests at the edges of the 256-request groups and of the list.  Enough
    requests reach positions 5-7 (the second launch) and enough reject."""
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=B, K=6, V=2056)
    inp = inputs.make_inputs(w, "cuda", seed=3)
    idx = _spread_requests(inp["temp"], 16, extra=(255, 256, 2047, 2048, 4095, 4096))
    tally, (_, _, _, acc, _) = _draft_and_verify(dsp, orc, inp, 9, idx, P.tol_for(w.dtype))
    n_tail, n_rej = int((acc >= 4).sum()), int((acc < w.K).sum())
    print(B, len(idx), tally, "reach position 5:", n_tail, "reject:", n_rej)
    assert n_tail >= 20 and n_rej >= 20
    assert tally.near_ties <= 1
    assert tally.draft_clean >= len(idx) - 1 and tally.verify_clean >= len(idx) - 1
    del inp
    torch.cuda.empty_cache()


def test_high_conc_pipeline_parity(dsp, orc, inputs):
    """Draft -> schedule -> verify of the scheduled prefixes over the dense
    target tensor ([B, K+1, V], offsets b (K+1)) at B=2048, V=131072, budget
    8192; the sampled requests span every scheduled length present."""
    w = inputs.WORKLOADS["high_conc"]
    inp = inputs.make_inputs(w, "cuda", seed=4)
    conf, _ = inputs.make_confidence(w, "cuda", seed=4)
    cn, ct = w.curve()
    L, offs, S = dsp.dspark_schedule(conf, w.budget, cn, ct)
    torch.cuda.synchronize()
    oL, ooffs, oS, n = orc.schedule(conf.cpu().numpy(), w.budget, np.array(cn), np.array(ct))
    np.testing.assert_array_equal(S.cpu().numpy(), oS)
    np.testing.assert_array_equal(L.cpu().numpy(), oL)
    np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
    Lc = oL
    assert int(ooffs[-1]) <= w.budget and Lc.min() < Lc.max()
    # one request per distinct length (up to 16), then the first and last
    idx = [0, w.B - 1]
    for v in sorted(set(Lc.tolist())):
        idx.append(int(np.nonzero(Lc == v)[0][0]))
    rng = np.random.default_rng(4)
    while len(set(idx)) < 16:
        idx.append(int(rng.integers(w.B)))
    idx = sorted(set(idx))
    dense = inputs.dense_offsets(w.B, w.K, "cuda")
    tally, _ = _draft_and_verify(dsp, orc, inp, 13, idx, P.tol_for(w.dtype), lengths=L,
                                 row_off=dense, target=inp["target"].reshape(-1, w.V))
    print(len(idx), sorted(set(Lc[idx].tolist())), tally)
    assert tally.near_ties <= 1 and tally.verify_clean >= len(idx) - 1
    del inp
    torch.cuda.empty_cache()


def test_conf_sched_pipeline_parity(dsp, orc, inputs):
    """Draft -> schedule -> ragged verify of the scheduled prefixes only."""
    w = inputs.WORKLOADS["conf_sched"]
    inp = inputs.make_inputs(w, "cuda", seed=3, with_target=False)
    conf, _ = inputs.make_confidence(w, "cuda", seed=3)
    cn, ct = w.curve()
    L, offs, S = dsp.dspark_schedule(conf, w.budget, cn, ct)
    torch.cuda.synchronize()
    oL, ooffs, oS, n = orc.schedule(conf.cpu().numpy(), w.budget, np.array(cn), np.array(ct))
    np.testing.assert_array_equal(S.cpu().numpy(), oS)
    np.testing.assert_array_equal(L.cpu().numpy(), oL)
    np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
    assert int(offs[-1]) <= w.budget
    target = inputs.ragged_target(w, inp["base"], L, offs, "cuda", seed=3)
    # one request per distinct scheduled length, the first and last, then
    # random ones up to 16
    idx = [0, w.B - 1]
    for v in sorted(set(oL.tolist())):
        idx.append(int(np.nonzero(oL == v)[0][0]))
    rng = np.random.default_rng(3)
    while len(set(idx)) < 16:
        idx.append(int(rng.integers(w.B)))
    idx = sorted(set(idx))
    tally, _ = _draft_and_verify(dsp, orc, inp, 9, idx, P.tol_for(w.dtype), lengths=L,
                                 row_off=offs, target=target)
    print(len(idx), sorted(set(oL[idx].tolist())), tally)
    assert tally.near_ties <= 1
    assert tally.draft_clean >= len(idx) - 1 and tally.verify_clean >= len(idx) - 1


@pytest.mark.parametrize("seed", range(6))
def test_schedule_parity_random(dsp, orc, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    K = int(rng.integers(1, 17))
    conf = rng.beta(5, 2, (B, K)).astype(np.float32)
    if seed == 1:
        conf[:] = 1.0  # all ties: order by k then b
    if seed == 2:
        conf[rng.random((B, K)) < 0.2] = 0.0
    for budget in (0, B - 1, B, B + 1, B + int(rng.integers(1, B * K + 1)), B * (K + 1) + 5):
        for curve in (None, (np.array([B + 3.0, B + 40.0]), np.array([1.0, 2.0]))):
            c = torch.from_numpy(conf).cuda()
            if curve is None:
                L, offs, S = dsp.dspark_schedule(c, budget)
                oL, ooffs, oS, _ = orc.schedule(conf, budget)
            else:
                L, offs, S = dsp.dspark_schedule(c, budget, curve[0].tolist(), curve[1].tolist())
                oL, ooffs, oS, _ = orc.schedule(conf, budget, curve[0].astype(np.float32)
                                                .astype(np.float64), curve[1])
            torch.cuda.synchronize()
            np.testing.assert_array_equal(S.cpu().numpy(), oS)
            np.testing.assert_array_equal(L.cpu().numpy(), oL)
            np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)


@pytest.mark.parametrize("B", [500, 700])
def test_schedule_longest_drafts(dsp, orc, B):
    """K = 64, the longest draft the scheduler takes: 32000 items (staged in LDS,
    keys in registers) and 44800 (rows walked in memory), with budgets that
    stop inside, at and past the items, under no curve, a curve whose rise
    stops the walk (a sort) and a flat curve (the threshold alone)."""
    K = 64
    rng = np.random.default_rng(B)
    conf = rng.beta(8, 1, (B, K)).astype(np.float32)
    conf[rng.random((B, K)) < 0.01] = 0.0
    c = torch.from_numpy(conf).cuda()
    curves = (None, ([float(B), float(B + 20000)], [1.0, 3.0]),
              ([float(B), float(B + B * K)], [2.0, 2.0]))
    for budget in (B + 777, B + 9000, B + 25000, B * (K + 1)):
        for curve in curves:
            if curve is None:
                L, offs, S = dsp.dspark_schedule(c, budget)
                oL, ooffs, oS, n = orc.schedule(conf, budget)
            else:
                L, offs, S = dsp.dspark_schedule(c, budget, curve[0], curve[1])
                oL, ooffs, oS, n = orc.schedule(conf, budget,
                                                np.float32(curve[0]).astype(np.float64),
                                                np.float32(curve[1]).astype(np.float64))
            torch.cuda.synchronize()
            print(B, budget, None if curve is None else curve[1], "taken", n)
            np.testing.assert_array_equal(S.cpu().numpy(), oS)
            np.testing.assert_array_equal(L.cpu().numpy(), oL)
            np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)


@pytest.mark.parametrize("B,K,extra,conf_kind", [
    (2048, 16, 12000, "beta"),    # 32768 items in registers, 12000 candidates: 16 per thread
    (2048, 16, 12000, "ones"),    # every S equal: the stop falls inside one run of ties
    (1500, 16, 9000, "levels"),   # few distinct confidences: many runs of equal S
    (3000, 16, 20000, "beta"),    # 48000 items: survival walk and 64-bit sort in memory
    (3000, 16, 20000, "levels"),
])
def test_schedule_large_parity(dsp, orc, B, K, extra, conf_kind):
    """Scheduler sizes past the small-batch paths: more than 8192 candidates
    sorted in LDS, more than 32768 items (keys and the candidate sort in
    workspace memory), and equal survival values around the stop rank, where
    the exact threshold key is chosen among keys that share the stop item's S.
    Each case runs without a curve, with a flat curve and with two sloped ones."""
    rng = np.random.default_rng(B + K + extra)
    if conf_kind == "beta":
        conf = rng.beta(5, 2, (B, K)).astype(np.float32)
    elif conf_kind == "ones":
        conf = np.ones((B, K), np.float32)
    else:
        conf = rng.choice(np.array([1.0, 0.75, 0.5], np.float32), (B, K))
    budget = B + extra
    c = torch.from_numpy(conf).cuda()
    curves = [None, ([float(B), float(budget)], [1.0, 1.0]),
              ([float(B + 64), float(B + 8192)], [1.0, 1.25]),
              ([float(B), float(B + 2048), float(B + 4096)], [1.0, 1.5, 4.0])]
    for curve in curves:
        if curve is None:
            L, offs, S = dsp.dspark_schedule(c, budget)
            oL, ooffs, oS, n = orc.schedule(conf, budget)
        else:
            cn = np.array(curve[0], np.float32)
            ct = np.array(curve[1], np.float32)
            L, offs, S = dsp.dspark_schedule(c, budget, cn.tolist(), ct.tolist())
            oL, ooffs, oS, n = orc.schedule(conf, budget, cn.astype(np.float64),
                                            ct.astype(np.float64))
        torch.cuda.synchronize()
        print(conf_kind, B, K, budget, None if curve is None else curve[1], "taken", n)
        np.testing.assert_array_equal(S.cpu().numpy(), oS)
        np.testing.assert_array_equal(L.cpu().numpy(), oL)
        np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)


def test_schedule_flat_curve_boundaries(dsp, orc):
    """A latency curve that is constant over every batch size the walk can
    reach ([B, B + D]) lets the scheduler take the threshold without sorting,
    when no taken S is small enough to vanish against the running total.
    Around that shortcut: survival values that do vanish in fp64 (the
    oracle's walk stops before D), a constant curve with a point inside the
    range, a dip inside the range, and a rise one token before B + D."""
    rng = np.random.default_rng(17)
    B, K = 100, 8
    cases = []
    # S = 1e-3^k: from k = 5 on, S < (B + sum S) 2^-53, so E + S == E
    tiny = np.full((B, K), 1e-3, np.float32)
    cases.append(("vanishing S", tiny, B + 700, [float(B), float(B + 700)], [2.0, 2.0], True))
    conf = rng.beta(5, 2, (B, K)).astype(np.float32)
    D = 500
    cases.append(("point inside", conf, B + D, [B - 5.0, B + 7.0, B + D + 3.0], [2.0, 2.0, 2.0],
                  False))
    cases.append(("dip inside", conf, B + D, [float(B), B + 250.0, float(B + D)], [1.0, 0.5, 1.0],
                  False))
    cases.append(("rise before B + D", conf, B + D, [float(B), B + D - 1.0, B + D + 100.0],
                  [1.0, 1.0, 3.0], False))
    c_t = {}
    for name, conf_c, budget, cn, ct, early in cases:
        key = id(conf_c)
        if key not in c_t:
            c_t[key] = torch.from_numpy(conf_c).cuda()
        cn32, ct32 = np.array(cn, np.float32), np.array(ct, np.float32)
        L, offs, S = dsp.dspark_schedule(c_t[key], budget, cn32.tolist(), ct32.tolist())
        torch.cuda.synchronize()
        oL, ooffs, oS, n = orc.schedule(conf_c, budget, cn32.astype(np.float64),
                                        ct32.astype(np.float64))
        print(name, "taken", n, "of", budget - B)
        np.testing.assert_array_equal(S.cpu().numpy(), oS)
        np.testing.assert_array_equal(L.cpu().numpy(), oL)
        np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
        if early:
            assert 0 < n < budget - B  # the oracle's walk stopped at a vanishing S


@pytest.mark.parametrize("jump", [1.05, 1.3, 2.0])
def test_schedule_stair_step_curve_parity(dsp, orc, inputs, jump):
    """A stair-step latency curve over the whole selectable range (49 points
    from B to the budget, a jump every 256 tokens, as a library GEMM's tiling
    gives): the early stop lands at a stair edge, bit-exact with the oracle."""
    w = inputs.WORKLOADS["conf_sched"]
    conf, _ = inputs.make_confidence(w, "cuda", seed=11)
    ns = np.arange(w.B, w.budget + 1, 64, dtype=np.float64)
    tau = (1.0 + 0.01 * (ns - w.B) / 64.0) * jump ** np.floor(ns / 256.0)
    cn, ct = ns.astype(np.float32), tau.astype(np.float32)
    L, offs, S = dsp.dspark_schedule(conf, w.budget, cn.tolist(), ct.tolist())
    torch.cuda.synchronize()
    oL, ooffs, oS, n = orc.schedule(conf.cpu().numpy(), w.budget, cn.astype(np.float64),
                                    ct.astype(np.float64))
    np.testing.assert_array_equal(S.cpu().numpy(), oS)
    np.testing.assert_array_equal(L.cpu().numpy(), oL)
    np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
    assert 0 < n <= w.budget - w.B


def test_schedule_high_conc_parity(dsp, orc, inputs):
    w = inputs.WORKLOADS["high_conc"]
    conf, _ = inputs.make_confidence(w, "cuda", seed=4)
    L, offs, S = dsp.dspark_schedule(conf, w.budget)
    torch.cuda.synchronize()
    oL, ooffs, oS, n = orc.schedule(conf.cpu().numpy(), w.budget)
    np.testing.assert_array_equal(L.cpu().numpy(), oL)
    np.testing.assert_array_equal(offs.cpu().numpy(), ooffs)
    assert n == w.budget - w.B


def test_verify_edge_cases(dsp, orc, inputs):
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=5, K=3, V=700, r=16)
    inp = inputs.make_inputs(w, "cuda", seed=21)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 2)
    target = inp["target"].reshape(-1, w.V)
    offs = torch.arange(w.B, dtype=torch.int64, device="cuda") * (w.K + 1)
    # L = 0 everywhere: bonus from row 1
    L0 = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    acc, nxt, rl, _ = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                        inp["W"], target, offs, inp["temp"], 2, L0)
    torch.cuda.synchronize()
    assert (acc == 0).all()
    for b in range(w.B):
        res = orc.verify_request(tok[b].cpu().numpy(), int(inp["prev"][b]),
                                 P.np32(inp["base"][b]), P.np32(inp["A"]), P.np32(inp["W"]),
                                 P.np32(target[b * (w.K + 1):b * (w.K + 1) + 1]), 0,
                                 float(inp["temp"][b]), 2, b)
        assert int(nxt[b]) == res["next_token"] or res["next_gap"] < P.NEAR_TIE
    # rows outside the target tensor: accepted 0, next -1, nothing read
    bad = offs.clone()
    bad[1] = 10**9
    bad[3] = -1
    acc, nxt, _, _ = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                       inp["W"], target, bad, inp["temp"], 2)
    acc2, nxt2, _, _ = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, bad, inp["temp"], 2,
                                         row_outputs=False)
    torch.cuda.synchronize()
    assert int(acc[1]) == 0 and int(nxt[1]) == -1
    assert int(acc[3]) == 0 and int(nxt[3]) == -1
    assert (nxt[[0, 2, 4]] >= 0).all()
    assert torch.equal(acc2, acc) and torch.equal(nxt2, nxt)


def test_two_streams_and_determinism(dsp, inputs):
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=32, K=4, V=20000, r=64)
    inp = inputs.make_inputs(w, "cuda", seed=8, with_target=False)
    ref = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 3)
    again = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 3)
    torch.cuda.synchronize()
    for x, y in zip(ref, again):
        assert torch.equal(x, y)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        o1 = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 3,
                                     stream=s1)
    with torch.cuda.stream(s2):
        o2 = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 4,
                                     stream=s2)
    torch.cuda.synchronize()
    for x, y in zip(ref, o1):
        assert torch.equal(x, y)
    o4 = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 4)
    torch.cuda.synchronize()
    for x, y in zip(o2, o4):
        assert torch.equal(x, y)


def test_gpu_chi_square_and_bitexact(dsp, orc):
    """10^6 requests (independent Philox streams): the first two emitted tokens
    follow the target's joint law; the first 1500 match the oracle bit for bit."""
    V, K, r, n, T, seed = 8, 2, 3, 1_000_000, 1.0, 77
    rng = np.random.default_rng(5)
    base = rng.normal(0, 1.2, (K, V)).astype(np.float32)
    A = rng.normal(0, 0.8, (V, r)).astype(np.float32)
    W = rng.normal(0, 0.8, (r, V)).astype(np.float32)
    t1 = (rng.normal(0, 1.0, V) + 0.7 * base[0]).astype(np.float32)
    t2 = rng.normal(0, 1.0, (V, V)).astype(np.float32)
    t3 = rng.normal(0, 1.0, (V, V, V)).astype(np.float32)

    def tgt(prefix):
        return [t1, t2[prefix[0]] if len(prefix) > 0 else None,
                t3[tuple(prefix[:2])] if len(prefix) > 1 else None][len(prefix)]

    dev = "cuda"
    g_base = torch.from_numpy(base).to(dev).expand(n, K, V).contiguous()
    g_A, g_W = torch.from_numpy(A).to(dev), torch.from_numpy(W).to(dev)
    prev = torch.full((n,), 3, dtype=torch.int32, device=dev)
    temp = torch.full((n,), T, dtype=torch.float32, device=dev)
    tok, logp, lse = dsp.dspark_draft_sample(g_base, g_A, g_W, prev, temp, seed)
    x = tok.long()
    rows = torch.stack([torch.from_numpy(t1).to(dev).expand(n, V),
                        torch.from_numpy(t2).to(dev)[x[:, 0]],
                        torch.from_numpy(t3).to(dev)[x[:, 0], x[:, 1]]], dim=1).contiguous()
    offs = torch.arange(n, dtype=torch.int64, device=dev) * (K + 1)
    acc, nxt, _, _ = dsp.dspark_verify(tok, prev, logp, lse, g_base, g_A, g_W,
                                       rows.view(-1, V), offs, temp, seed)
    torch.cuda.synchronize()
    tok_c, acc_c, nxt_c = tok.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()
    # bit-exact against the oracle on a prefix of the requests
    m = 1500
    o_tok, o_logp, o_lse, o_gap = orc.draft_batch(np.broadcast_to(base, (m, K, V)), A, W,
                                                  np.full(m, 3, np.int32), np.full(m, T, np.float32),
                                                  seed)
    o_rows = rows[:m].cpu().numpy().reshape(-1, V)
    orv = orc.verify_batch(o_tok, np.full(m, 3, np.int32), np.broadcast_to(base, (m, K, V)), A, W,
                           o_rows, np.arange(m, dtype=np.int64) * (K + 1), None,
                           np.full(m, T, np.float32), seed)
    near = 0
    for b in range(m):
        if (tok_c[b] != o_tok[b]).any():
            assert o_gap[b].min() < P.NEAR_TIE
            near += 1
            continue
        if acc_c[b] != orv["accepted"][b] or nxt_c[b] != orv["next_token"][b]:
            assert min(orv["accept_gap"][b], orv["next_gap"][b]) < P.NEAR_TIE
            near += 1
    assert near <= 3
    # law of the first two emitted tokens
    z1 = np.where(acc_c >= 1, tok_c[:, 0], nxt_c)
    z2 = np.where(acc_c >= 2, tok_c[:, 1], np.where(acc_c == 1, nxt_c, -1))
    need = np.nonzero(z2 < 0)[0]
    crng = np.random.default_rng(9)
    for a in range(V):
        sel = need[z1[need] == a]
        if len(sel):
            z2[sel] = crng.choice(V, size=len(sel), p=orc.target_probs(t2[a], T))
    joint = orc.target_joint(tgt, T, V, 2)
    expect = np.array([[joint[(a, b)] for b in range(V)] for a in range(V)]) * n
    counts = np.zeros((V, V))
    np.add.at(counts, (z1, z2), 1)
    chi = ((counts - expect) ** 2 / expect).sum()
    assert stats.chi2.sf(chi, V * V - 1) > 1e-3
    # acceptance rate at position 1 against 1 - TV
    pd = orc.draft_probs(base[0], A, W, 3, T)
    pt = orc.target_probs(t1, T)
    p_acc = np.minimum(pd, pt).sum()
    rate = (acc_c >= 1).mean()
    assert abs(rate - p_acc) < 5 * np.sqrt(p_acc * (1 - p_acc) / n)


def test_profile_session_counts_and_times_launches(dsp, inputs):
    """The event-timing session sees every launch of the kernels it was asked
    for (K draft strips and combines per call), times them on their stream, and
    leaves other kernels alone."""
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=64, K=3, V=8192, r=256)
    inp = inputs.make_inputs(w, "cuda", seed=12, with_target=False)
    dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 5)
    torch.cuda.synchronize()
    dsp.dspark_profile_begin(("draft_strip", "draft_combine"), max_launches=64)
    for _ in range(2):
        dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 5)
    res = dsp.dspark_profile_end()
    assert res["draft_strip"][1:] == (2 * w.K, 2 * w.K)
    assert res["draft_combine"][1:] == (2 * w.K, 2 * w.K)
    assert all(res[k][0] > 0.0 for k in ("draft_strip", "draft_combine"))
    assert res["verify_rows"] == (0.0, 0, 0)
    # a second session after the first one closed starts from zero; launches
    # beyond the event pool are counted but not timed
    dsp.dspark_profile_begin(("draft_strip",), max_launches=2)
    dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], 5)
    res = dsp.dspark_profile_end()
    assert res["draft_strip"][1:] == (w.K, 2)
