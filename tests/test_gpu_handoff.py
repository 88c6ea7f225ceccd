"""GPU parity of the rank-256 draft kernel's load balancing, and of the
residual kernel with a long residual list.

With eight wavefronts per workgroup, a greedy wavefront draws the last tile of
every strip but the final one for the sampled wavefronts of a loaded SIMD
(wavefronts h + 2 and h + 6 for helper h in {0, 1}).  These cases place
exactly n_greedy greedy requests at random positions, so the visit order
(greedy first) puts chosen wavefronts in each role, with V large enough that
every workgroup walks several strips.  The compared requests are the ones in
the helped wavefronts' slots (greedy lanes of a mixed helped wavefront
included) and a few from the others.
"""
import numpy as np
import pytest
import torch

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


def _visit_order(temp):
    """The strip kernels' visit order: greedy requests first, then sampled,
    each kind in request order, with every group of 256 slots taking its share
    floor(n_greedy (g + 1) 256 / B) - floor(n_greedy g 256 / B) of the greedy
    ones (first in the group)."""
    t = temp.cpu().numpy()
    B = len(t)
    greedy = [b for b in range(B) if not t[b] > 0]
    sampled = [b for b in range(B) if t[b] > 0]
    ng = len(greedy)
    order = []
    for start in range(0, B, 256):
        end = min(start + 256, B)
        q0, q1 = ng * start // B, ng * end // B
        order += greedy[q0:q1] + sampled[start - q0:end - q1]
    assert sorted(order) == list(range(B))
    return order


# (B, V, K, n_greedy): 64 -> both helpers; 70 -> helper 0 serves a mixed
# wavefront 2; 40 -> only helper 0 (wavefront 1 mixed); 96 -> only helper 1;
# B = 200 -> wavefront 6 half active and 7 inactive (helper 0 only);
# B = 300 -> a second request group of 44 slots; B = 512 -> two groups, each
# with its share of the greedy requests; 0 -> every wavefront samples (no
# helper); 256 -> every wavefront greedy (argmax epilogue only, nothing handed)
CASES = [
    (256, 70016, 3, 64),
    (256, 40064, 2, 0),
    (256, 40064, 2, 256),
    (200, 66048, 2, 64),
    (256, 66048, 2, 70),
    (256, 66048, 2, 40),
    (256, 66048, 2, 96),
    (300, 40064, 3, 70),
    (512, 40064, 2, 64),
]


@pytest.mark.parametrize("B,V,K,n_greedy", CASES)
def test_rank256_handoff_parity(dsp, orc, inputs, B, V, K, n_greedy):
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=B, K=K, V=V)
    inp = inputs.make_inputs(w, "cuda", seed=11, with_target=False)
    rng = np.random.default_rng(B + V + n_greedy)
    t = np.where(rng.random(B) < 0.5, 0.7, 1.0).astype(np.float32)
    t[rng.permutation(B)[:n_greedy]] = 0.0
    inp["temp"] = torch.from_numpy(t).to("cuda")
    order = _visit_order(inp["temp"])
    # slots of wavefronts 2, 3, 6 and 7 of every request group, six per wavefront
    idx = set()
    for g in range((B + 255) // 256):
        for wv in (2, 3, 6, 7):
            slots = [s for s in range((g * 8 + wv) * 32, (g * 8 + wv + 1) * 32) if s < B]
            for s in slots[:: max(1, len(slots) // 6)][:6]:
                idx.add(order[s])
        for wv in (0, 1, 4, 5):
            s = (g * 8 + wv) * 32 + 5
            if s < B:
                idx.add(order[s])
    idx = sorted(idx)
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], 7)
    torch.cuda.synchronize()
    ora = P.oracle_draft(orc, inp, idx, 7)
    tally = P.Tally()
    P.compare_draft(tok.cpu().numpy(), logp.cpu().numpy(), lse.cpu().numpy(), ora,
                    inp["temp"].cpu().numpy(), P.tol_for(w.dtype), tally)
    print(B, V, K, n_greedy, len(idx), tally)
    assert tally.near_ties <= 1
    assert tally.draft_clean >= len(idx) - 1
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_sampled", [140, 170, 185])
def test_residual_handoff_parity(dsp, orc, inputs, n_sampled):
    """The residual strip kernel with a long residual list: with a target far
    from the draft most sampled requests reject at their first row, so the list
    holds about n_sampled requests and fills five to six of the eight
    wavefronts, over several strips per workgroup.  Every sampled request's
    verify result is compared with the oracle's on the GPU's drafted tokens."""
    B, V, K = 256, 70016, 3
    w = inputs.resized(inputs.WORKLOADS["long_draft"], B=B, K=K, V=V, noise_lo=6.0, noise_hi=6.0)
    inp = inputs.make_inputs(w, "cuda", seed=13)
    rng = np.random.default_rng(n_sampled)
    t = np.zeros(B, np.float32)
    t[rng.permutation(B)[:n_sampled]] = rng.choice(np.float32([0.7, 1.0]), n_sampled)
    inp["temp"] = torch.from_numpy(t).to("cuda")
    seed = 9
    tok, logp, lse = dsp.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                             inp["temp"], seed)
    target = inp["target"].reshape(-1, V)
    offs = torch.arange(B, dtype=torch.int64, device="cuda") * (K + 1)
    acc, nxt, rl, rr = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, offs, inp["temp"], seed)
    acc2, nxt2, _, _ = dsp.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                         inp["W"], target, offs, inp["temp"], seed,
                                         row_outputs=False)
    torch.cuda.synchronize()
    assert torch.equal(acc2, acc) and torch.equal(nxt2, nxt)
    idx = [int(b) for b in np.nonzero(t > 0)[0]]
    acc_np = acc.cpu().numpy()
    assert (acc_np[idx] < K).sum() >= 0.9 * len(idx)  # the list is about n_sampled long
    tok_np = tok.cpu().numpy()
    rows = {b: P.np32(target[b * (K + 1):(b + 1) * (K + 1)]) for b in idx}
    orv = P.oracle_verify(orc, inp, idx, {b: tok_np[b] for b in idx}, rows, {b: K for b in idx},
                          seed)
    tally = P.compare_verify(acc_np, nxt.cpu().numpy(), rl.cpu().numpy(), rr.cpu().numpy(),
                             offs.cpu().numpy(), orv, P.tol_for(w.dtype))
    print(n_sampled, len(idx), tally)
    assert tally.near_ties <= 1
    assert tally.verify_clean >= len(idx) - 1
    del inp
    torch.cuda.empty_cache()
