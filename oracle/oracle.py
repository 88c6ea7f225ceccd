"""Python binding of the CPU oracle (``oracle/dspark_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg use this module.  The HIP product path never
imports it.  Inputs are numpy arrays; bf16 inputs are widened to fp32 by the
caller (exactly).  See the C source for the definitions and their sources.

Also holds the exact enumeration used by the losslessness pins: for tiny V
and K it sums, over every draft sequence, the probability that verification
emits each token tuple (the textbook accept / residual / bonus rule written
as probabilities) and completes the tuple with target draws.
"""
from __future__ import annotations

import ctypes
import itertools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

TAG_DRAFT, TAG_ACCEPT, TAG_RESAMPLE = 0, 1, 2
BRANCH_BONUS, BRANCH_RESIDUAL, BRANCH_FALLBACK = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
            "-fno-fast-math", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_F = ctypes.c_float
_D = ctypes.c_double


def _declare(L):
    L.oracle_philox4x32_10.argtypes = [_P, _P, _P]
    L.oracle_philox4x32_10.restype = None
    L.oracle_uniform.argtypes = [_U64, _U32, _U32, _U32, _U32]
    L.oracle_uniform.restype = _F
    L.oracle_gumbel.argtypes = [_U64, _U32, _U32, _U32, _U32]
    L.oracle_gumbel.restype = _F
    L.oracle_draft_probs.argtypes = [_P, _P, _P, _I, _I, _I, _F, _P]
    L.oracle_draft_probs.restype = None
    L.oracle_target_probs.argtypes = [_P, _I, _F, _P]
    L.oracle_target_probs.restype = None
    L.oracle_draft_request.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_int32, _F, _U64, _U32,
                                       _P, _P, _P, _P]
    L.oracle_draft_request.restype = None
    L.oracle_draft_batch.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _U64, _P, _P, _P, _P]
    L.oracle_draft_batch.restype = None
    L.oracle_verify_request.argtypes = [_P, ctypes.c_int32, _P, _P, _P, _I, _I, _I, _P, _I, _F,
                                        _U64, _U32, _P, _P, _P, _P, _P, _P, _P]
    L.oracle_verify_request.restype = None
    L.oracle_verify_batch.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _U64,
                                      _P, _P, _P, _P, _P, _P, _P]
    L.oracle_verify_batch.restype = None
    L.oracle_curve_tau.argtypes = [_P, _P, _I, _D]
    L.oracle_curve_tau.restype = _D
    L.oracle_schedule.argtypes = [_P, _I, _I, ctypes.c_int64, _P, _P, _I, _P, _P, _P]
    L.oracle_schedule.restype = _I


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_P)


# --------------------------------------------------------------------------- RNG
def philox4x32_10(counter, key):
    """Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words."""
    c, cp = _c(counter, np.uint32)
    k, kp = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(cp, kp, out.ctypes.data_as(_P))
    return out


def uniform(seed, b, pos, tag, v):
    return np.float32(lib().oracle_uniform(seed, b, pos, tag, v))


def gumbel(seed, b, pos, tag, v):
    return np.float32(lib().oracle_gumbel(seed, b, pos, tag, v))


# ------------------------------------------------------------------ probabilities
def draft_probs(base_k, A, W, prev, T):
    base_k, bp = _c(base_k, np.float32)
    A, ap = _c(A, np.float32)
    W, wp = _c(W, np.float32)
    V = base_k.shape[0]
    r = A.shape[1]
    p = np.zeros(V, np.float64)
    lib().oracle_draft_probs(bp, ap, wp, V, r, int(prev), float(T), p.ctypes.data_as(_P))
    return p


def target_probs(t_row, T):
    t_row, tp = _c(t_row, np.float32)
    p = np.zeros(t_row.shape[0], np.float64)
    lib().oracle_target_probs(tp, t_row.shape[0], float(T), p.ctypes.data_as(_P))
    return p


# ------------------------------------------------------------------------- draft
def draft_request(base, A, W, prev0, T, seed, b):
    """One request: base [K, V] -> tokens [K], logp [K], lse [K], gap [K]."""
    base, bp = _c(base, np.float32)
    A, ap = _c(A, np.float32)
    W, wp = _c(W, np.float32)
    K, V = base.shape
    r = A.shape[1]
    tok = np.zeros(K, np.int32)
    logp = np.zeros(K, np.float32)
    lse = np.zeros(K, np.float32)
    gap = np.zeros(K, np.float64)
    lib().oracle_draft_request(bp, ap, wp, V, r, K, int(prev0), float(T), int(seed), int(b),
                               tok.ctypes.data_as(_P), logp.ctypes.data_as(_P),
                               lse.ctypes.data_as(_P), gap.ctypes.data_as(_P))
    return tok, logp, lse, gap


def draft_batch(base, A, W, prev0, T, seed):
    """All requests: base [B, K, V] -> tokens, logp, lse, gap, each [B, K]."""
    base, bp = _c(base, np.float32)
    A, ap = _c(A, np.float32)
    W, wp = _c(W, np.float32)
    prev0, pp = _c(prev0, np.int32)
    T, tp = _c(T, np.float32)
    B, K, V = base.shape
    r = A.shape[1]
    tok = np.zeros((B, K), np.int32)
    logp = np.zeros((B, K), np.float32)
    lse = np.zeros((B, K), np.float32)
    gap = np.zeros((B, K), np.float64)
    lib().oracle_draft_batch(bp, ap, wp, B, K, V, r, pp, tp, int(seed), tok.ctypes.data_as(_P),
                             logp.ctypes.data_as(_P), lse.ctypes.data_as(_P),
                             gap.ctypes.data_as(_P))
    return tok, logp, lse, gap


# ------------------------------------------------------------------------ verify
def verify_request(tokens, prev0, base, A, W, target_rows, L, T, seed, b):
    """One request.  target_rows [L+1, V] are the request's verify rows."""
    tokens, tkp = _c(tokens, np.int32)
    base, bp = _c(base, np.float32)
    A, ap = _c(A, np.float32)
    W, wp = _c(W, np.float32)
    target_rows, trp = _c(target_rows, np.float32)
    K, V = base.shape
    r = A.shape[1]
    assert target_rows.shape[0] >= L + 1
    acc = np.zeros(1, np.int32)
    nxt = np.zeros(1, np.int32)
    lse_t = np.zeros(L + 1, np.float32)
    ratio = np.zeros(L + 1, np.float32)
    ag = np.zeros(1, np.float64)
    ng = np.zeros(1, np.float64)
    br = np.zeros(1, np.int32)
    lib().oracle_verify_request(tkp, int(prev0), bp, ap, wp, V, r, K, trp, int(L), float(T),
                                int(seed), int(b), acc.ctypes.data_as(_P), nxt.ctypes.data_as(_P),
                                lse_t.ctypes.data_as(_P), ratio.ctypes.data_as(_P),
                                ag.ctypes.data_as(_P), ng.ctypes.data_as(_P),
                                br.ctypes.data_as(_P))
    return dict(accepted=int(acc[0]), next_token=int(nxt[0]), row_lse_t=lse_t,
                row_logratio=ratio, accept_gap=float(ag[0]), next_gap=float(ng[0]),
                branch=int(br[0]))


def verify_batch(tokens, prev0, base, A, W, target, row_offsets, lengths, T, seed):
    """All requests over ragged target rows [rows, V]; row_offsets [B] int64."""
    tokens, tkp = _c(tokens, np.int32)
    prev0, pp = _c(prev0, np.int32)
    base, bp = _c(base, np.float32)
    A, ap = _c(A, np.float32)
    W, wp = _c(W, np.float32)
    target, trp = _c(target, np.float32)
    row_offsets, rop = _c(row_offsets, np.int64)
    T, tp = _c(T, np.float32)
    B, K, V = base.shape
    r = A.shape[1]
    if lengths is None:
        lp = None
    else:
        lengths, lp = _c(lengths, np.int32)
    rows = target.shape[0]
    acc = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    lse_t = np.zeros(rows, np.float32)
    ratio = np.zeros(rows, np.float32)
    ag = np.zeros(B, np.float64)
    ng = np.zeros(B, np.float64)
    br = np.zeros(B, np.int32)
    lib().oracle_verify_batch(tkp, pp, bp, ap, wp, B, K, V, r, trp, rop, lp, tp, int(seed),
                              acc.ctypes.data_as(_P), nxt.ctypes.data_as(_P),
                              lse_t.ctypes.data_as(_P), ratio.ctypes.data_as(_P),
                              ag.ctypes.data_as(_P), ng.ctypes.data_as(_P),
                              br.ctypes.data_as(_P))
    return dict(accepted=acc, next_token=nxt, row_lse_t=lse_t, row_logratio=ratio,
                accept_gap=ag, next_gap=ng, branch=br)


# ---------------------------------------------------------------------- schedule
def curve_tau(curve_n, curve_tau_, N):
    cn, cnp = _c(curve_n, np.float64)
    ct, ctp = _c(curve_tau_, np.float64)
    return lib().oracle_curve_tau(cnp, ctp, len(cn), float(N))


def schedule(conf, budget, curve_n=None, curve_tau_=None):
    """conf [B, K] -> lengths [B], row_offsets [B+1], survival [B, K], n_selected."""
    conf, cp = _c(conf, np.float32)
    B, K = conf.shape
    if curve_n is None:
        cnp = ctp = None
        npts = 0
    else:
        cn, cnp = _c(curve_n, np.float64)
        ct, ctp = _c(curve_tau_, np.float64)
        npts = len(cn)
    lengths = np.zeros(B, np.int32)
    offs = np.zeros(B + 1, np.int64)
    surv = np.zeros((B, K), np.float32)
    n = lib().oracle_schedule(cp, B, K, int(budget), cnp, ctp, npts, lengths.ctypes.data_as(_P),
                              offs.ctypes.data_as(_P), surv.ctypes.data_as(_P))
    return lengths, offs, surv, int(n)


# ------------------------------------------------------------ exact enumeration
def _residual_mass(pt, pd):
    """Unnormalised residual law after a rejection: max(0, p_t - p_d)."""
    return np.maximum(pt - pd, 0.0)


def emitted_distribution(base, A, W, prev0, T, target_fn, n_out=None):
    """Exact distribution of the first ``n_out`` (default K+1) emitted tokens.

    base [K, V] draft base logits; target_fn(prefix_tuple) -> target logits row
    [V] for the position after ``prefix_tuple``.  Draft sequences are
    enumerated with probability prod_k p_d(x_k | x_{k-1}); verification is
    the accept / residual / bonus rule written as probabilities; tokens after
    the emitted ones are completed with target draws.  Returns a dict mapping
    token tuples to probabilities.
    """
    K, V = base.shape
    n_out = K + 1 if n_out is None else n_out
    pt_cache = {}

    def p_t(prefix):
        if prefix not in pt_cache:
            pt_cache[prefix] = target_probs(target_fn(prefix), T)
        return pt_cache[prefix]

    pd_cache = {}

    def p_d(k, prev):
        key = (k, prev)
        if key not in pd_cache:
            pd_cache[key] = draft_probs(base[k], A, W, prev, T)
        return pd_cache[key]

    out = {}

    def complete(prefix, mass):
        if len(prefix) >= n_out:
            key = prefix[:n_out]
            out[key] = out.get(key, 0.0) + mass
            return
        pt = p_t(prefix)
        for v in range(V):
            if pt[v] > 0.0:
                complete(prefix + (v,), mass * pt[v])

    for x in itertools.product(range(V), repeat=K):
        prob_x = 1.0
        prev = prev0
        for k in range(K):
            prob_x *= p_d(k, prev)[x[k]]
            prev = x[k]
        if prob_x == 0.0:
            continue
        still = prob_x  # probability that positions 1..a were all accepted
        for a in range(K + 1):
            if a == K:  # bonus from row K+1
                pt = p_t(tuple(x))
                for v in range(V):
                    if pt[v] > 0.0:
                        complete(tuple(x) + (v,), still * pt[v])
                break
            j = a + 1
            prev = prev0 if j == 1 else x[j - 2]
            pd = p_d(j - 1, prev)
            pt = p_t(tuple(x[: j - 1]))
            xj = x[j - 1]
            ratio = min(1.0, pt[xj] / pd[xj])
            rej = still * (1.0 - ratio)
            if rej > 0.0:
                res = _residual_mass(pt, pd)
                tot = res.sum()
                res = res / tot if tot > 0.0 else pt
                for v in range(V):
                    if res[v] > 0.0:
                        complete(tuple(x[: j - 1]) + (v,), rej * res[v])
            still *= ratio
            if still == 0.0:
                break
    return out


def target_joint(target_fn, T, V, n_out):
    """prod_j p_t(z_j | z_<j) for every tuple of length n_out."""
    out = {}

    def rec(prefix, mass):
        if len(prefix) == n_out:
            out[prefix] = mass
            return
        pt = target_probs(target_fn(prefix), T)
        for v in range(V):
            if pt[v] > 0.0:
                rec(prefix + (v,), mass * pt[v])

    rec((), 1.0)
    return out
