"""Helpers shared by the GPU parity tests: run the oracle on a subset of
requests and compare with the HIP path element by element.

Comparison rules (from the hot path's parity bar):
* tokens, accepted lengths, next tokens and scheduled lengths are bit-exact,
  except near-ties: where the oracle's top-2 perturbed values (or the accept
  test's |log u - log ratio|) are within 1e-5, the two sides may legitimately
  differ; such cases are counted and the rest of that request is excluded;
* log-normalisers, log-probabilities and log-ratios agree within a tolerance
  of 2e-3 (bf16 inputs) or 1e-5 (fp32 inputs) relative to max(1, |value|).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

NEAR_TIE = 1e-5


def tol_for(dtype) -> float:
    return 2e-3 if dtype == torch.bfloat16 else 1e-5


def np32(t) -> np.ndarray:
    """Exact widening of a (bf16 or fp32) tensor to a float32 numpy array."""
    return t.detach().to("cpu").float().numpy()


def close(a, b, tol) -> bool:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    finite = np.isfinite(a) & np.isfinite(b)
    diff = np.abs(np.where(finite, a, 0.0) - np.where(finite, b, 0.0))
    ok = both_inf | (finite & (diff <= tol * np.maximum(1.0, np.abs(np.where(finite, b, 0.0)))))
    return bool(ok.all())


class Tally:
    """compared: draft positions and verify requests that matched; near_ties:
    divergences excused by a near-tie; draft_clean / verify_clean: requests
    whose whole draft (every position) / verify result matched."""

    def __init__(self):
        self.near_ties = 0
        self.compared = 0
        self.draft_clean = 0
        self.verify_clean = 0

    def __repr__(self):
        return (f"Tally(compared={self.compared}, near_ties={self.near_ties}, "
                f"draft_clean={self.draft_clean}, verify_clean={self.verify_clean})")


def workers() -> int:
    """Oracle threads: the oracle is single-threaded C called through ctypes
    (which releases the GIL), so independent requests run side by side, at
    most 16 at a time."""
    return max(1, min(16, os.cpu_count() or 1))


def _map(fn, idx):
    idx = list(idx)
    if len(idx) <= 1:
        return {b: fn(b) for b in idx}
    with ThreadPoolExecutor(min(workers(), len(idx))) as ex:
        return dict(zip(idx, ex.map(fn, idx)))


def oracle_draft(orc, inp, idx, seed):
    """Oracle draft for the requests in idx (global request indices)."""
    A = np32(inp["A"])
    W = np32(inp["W"])
    prev = inp["prev"].cpu().numpy()
    temp = inp["temp"].cpu().numpy()
    bases = {b: np32(inp["base"][b]) for b in idx}
    return _map(lambda b: orc.draft_request(bases[b], A, W, int(prev[b]), float(temp[b]), seed,
                                            int(b)), idx)


def compare_draft(gpu_tok, gpu_logp, gpu_lse, ora, temp, tol, tally=None):
    """Compare GPU draft rows with oracle results {b: (tok, logp, lse, gap)}.
    Returns the set of requests whose whole draft matched (no divergence)."""
    tally = tally or Tally()
    clean = set()
    for b, (tok, logp, lse, gap) in ora.items():
        K = len(tok)
        diverged = False
        for k in range(K):
            if int(gpu_tok[b, k]) != int(tok[k]):
                assert gap[k] < NEAR_TIE, (
                    f"draft token mismatch b={b} k={k}: gpu={int(gpu_tok[b, k])} "
                    f"oracle={int(tok[k])} top-2 gap={gap[k]:.3g}")
                tally.near_ties += 1
                diverged = True
                break
            assert close(gpu_lse[b, k], lse[k], tol), (b, k, float(gpu_lse[b, k]), float(lse[k]))
            assert close(gpu_logp[b, k], logp[k], tol), (b, k, float(gpu_logp[b, k]), float(logp[k]))
            tally.compared += 1
        if not diverged:
            clean.add(b)
            tally.draft_clean += 1
    return clean


def oracle_verify(orc, inp, idx, tokens, target_rows, lengths, seed):
    """Oracle verify for requests idx.  tokens: {b: int32[K]} (oracle draft);
    target_rows: {b: float32[L_b+1, V]}; lengths: {b: L_b}."""
    A = np32(inp["A"])
    W = np32(inp["W"])
    prev = inp["prev"].cpu().numpy()
    temp = inp["temp"].cpu().numpy()
    bases = {b: np32(inp["base"][b]) for b in idx}
    return _map(lambda b: orc.verify_request(tokens[b], int(prev[b]), bases[b], A, W,
                                             target_rows[b], int(lengths[b]), float(temp[b]),
                                             seed, int(b)), idx)


def compare_verify(gpu_acc, gpu_next, gpu_lse_rows, gpu_ratio_rows, row_off, ora, tol,
                   tally=None):
    tally = tally or Tally()
    for b, res in ora.items():
        L = len(res["row_lse_t"]) - 1
        ro = int(row_off[b])
        assert close(gpu_lse_rows[ro:ro + L + 1], res["row_lse_t"], tol), (
            b, gpu_lse_rows[ro:ro + L + 1], res["row_lse_t"])
        assert close(gpu_ratio_rows[ro:ro + L], res["row_logratio"][:L], tol), (
            b, gpu_ratio_rows[ro:ro + L], res["row_logratio"][:L])
        if int(gpu_acc[b]) != res["accepted"]:
            assert res["accept_gap"] < NEAR_TIE, (
                f"accepted mismatch b={b}: gpu={int(gpu_acc[b])} oracle={res['accepted']} "
                f"gap={res['accept_gap']:.3g}")
            tally.near_ties += 1
            continue
        if int(gpu_next[b]) != res["next_token"]:
            assert res["next_gap"] < NEAR_TIE or res["accept_gap"] < NEAR_TIE, (
                f"next token mismatch b={b}: gpu={int(gpu_next[b])} oracle={res['next_token']} "
                f"gap={res['next_gap']:.3g}")
            tally.near_ties += 1
            continue
        tally.compared += 1
        tally.verify_clean += 1
    return tally
