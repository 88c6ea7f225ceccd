"""Benchmark of the draft -> schedule -> verify hot path on one MI355X.

One step = one pass of the whole hot path over one batch of the long-draft
workload (B=256 requests, K=16 draft positions, V=151936, rank 256, bf16,
temperatures mixed over {0, 0.7, 1}): Markov-head draft of all K tokens,
confidence scheduling with a budget that admits every drafted token (the
workload verifies the full draft), and verification of every drafted token.
Inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line (metric: drafted-and-verified tokens per second).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
VALU_PEAK_TOPS = 39.3        # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz vector-ALU lane operations
METRIC = "draft+verify tokens/s at B=256,K=16,V=151936; % of HBM / MFMA roofline"
# Files whose contents define the dominant kernel; the stored PMC traffic figure
# is only reported while their hash matches the one it was measured with.
DOMINANT_SOURCES = ("draft_mfma.hip", "common.hpp", "kernels.hpp")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "draft_strip_mfma_long_draft_pmc.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_draft")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=24)
    ap.add_argument("--markov-vs-parallel", action="store_true",
                    help="also time the draft with the Markov head against parallel drafting "
                         "(no transition factors) at K = 4 and K = 16")
    ap.add_argument("--sps-curve", action="store_true",
                    help="also measure a stair-step step-latency curve (a bf16 GEMM over N batch "
                         "tokens) and schedule the confidence workload with it: greedy early stop "
                         "against a global search over N, and with the budget taken from "
                         "confidences two steps back")
    ap.add_argument("--calibration", action="store_true",
                    help="also calibrate a synthetic, over-confident confidence head against "
                         "the acceptance outcomes of dspark_verify with sequential temperature "
                         "scaling, and report the expected calibration error before and after")
    ap.add_argument("--no-extras", action="store_true",
                    help="report the headline measurement only (by default the line also "
                         "carries --markov-vs-parallel, --sps-curve, --calibration and short "
                         "timed runs of the other workloads, measured after the headline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain copy kernel (torch.neg, fp32) of this many MiB before "
                         "warmup, as the reference for HBM counter scaling")
    return ap.parse_args()


def dominant_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, "draft_sampling_verification_04_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_counters():
    """Per-launch figures of the dominant kernel from the committed PMC summary
    (HBM bytes, VALU wave instructions, transcendental ones), or None when the
    kernel's sources changed since the counters were taken."""
    keys = ("source_hash", "traffic_bytes_per_launch", "valu_instructions_per_launch",
            "valu_trans_instructions_per_launch")
    try:
        with open(PMC_SUMMARY) as f:
            fields = dict(l.split(":", 1) for l in f.read().splitlines() if l.startswith(keys))
    except (OSError, ValueError):
        return None
    if fields.get("source_hash", "").strip() != dominant_source_hash():
        return None
    try:
        return {k: int(fields[k].strip()) for k in keys[1:]}
    except (KeyError, ValueError):
        return None


def alu_view(stored, launch_s):
    """The dominant kernel against the vector-ALU peak, from the committed
    counters: VALU lane-operations issued per second (wave instructions x 64
    lanes, a transcendental counted twice: it issues at half rate) over the
    peak of 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-ops/s.  This
    is issued work, not an algorithmic count; null when the counters are
    stale."""
    if not stored:
        return None
    ops = 64 * (stored["valu_instructions_per_launch"] + stored["valu_trans_instructions_per_launch"])
    rate = ops / launch_s
    return {"lane_ops_per_launch": ops, "achieved": round(rate / 1e12, 2), "peak": VALU_PEAK_TOPS,
            "unit": "T lane-ops/s", "frac": round(rate / 1e12 / VALU_PEAK_TOPS, 4)}


def verify_position_launches(K):
    """Position ranges of the verify-rows launches when no per-row outputs are
    asked for (the schedule dspark_verify documents): 1..min(4, K+1), then
    5..K+1."""
    out = [(1, min(4, K + 1))]
    if K + 1 > 4:
        out.append((5, K + 1))
    return out


def target_rows_read(lengths, accepted, K):
    """Target rows verify reads without per-row outputs: request b takes part
    in a launch over positions j0..j1 while rows 1..j0-1 were all accepted
    (accepted[b] >= j0 - 1), and reads its rows j0..min(j1, L_b + 1) there."""
    n = 0
    for L_b, a_b in zip(lengths, accepted):
        for j0, j1 in verify_position_launches(K):
            if j0 > L_b + 1 or a_b < j0 - 1:
                break
            n += min(j1, L_b + 1) - j0 + 1
    return n


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(w, inp, seed, n_req, target, row_off, lengths, gpu):
    """Time the oracle (single-threaded C) on n_req requests of the same
    workload: full draft of K tokens plus verification of the request's
    scheduled prefix over the same target rows the GPU read.  The oracle's
    results are then compared with the GPU's (gpu = tokens, accepted, next
    token) request by request: a divergence is allowed only where the oracle
    reports a near-tie (top-2 perturbed values, or |log u - log ratio|,
    within 1e-5)."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import numpy as np
    import oracle as orc

    A = inp["A"].float().cpu().numpy()
    W = inp["W"].float().cpu().numpy()
    prev = inp["prev"].cpu().numpy()
    temp = inp["temp"].cpu().numpy()
    ro = row_off.cpu().numpy()
    Ls = lengths.cpu().numpy()
    g_tok, g_acc, g_nxt = (t.cpu().numpy() for t in gpu)
    # sample requests with T > 0 (the expensive, sampled case) first
    order = sorted(range(w.B), key=lambda b: (temp[b] == 0.0, b))[:n_req]
    t_total = 0.0
    near = matched = 0
    for b in order:
        base = inp["base"][b].float().cpu().numpy()
        rows = target[int(ro[b]):int(ro[b]) + int(Ls[b]) + 1].float().cpu().numpy()
        t0 = time.perf_counter()
        tok, _, _, gap = orc.draft_request(base, A, W, int(prev[b]), float(temp[b]), seed, b)
        v = orc.verify_request(tok, int(prev[b]), base, A, W, rows, int(Ls[b]), float(temp[b]),
                               seed, b)
        t_total += time.perf_counter() - t0
        if (g_tok[b] != tok).any():
            k = int(np.nonzero(g_tok[b] != tok)[0][0])
            if not gap[k] < 1e-5:
                raise AssertionError(f"oracle/GPU draft mismatch at request {b}, position {k}")
            near += 1
        elif g_acc[b] != v["accepted"] or g_nxt[b] != v["next_token"]:
            if not min(v["accept_gap"], v["next_gap"]) < 1e-5:
                raise AssertionError(f"oracle/GPU verify mismatch at request {b}")
            near += 1
        else:
            matched += 1
    tokens = n_req * w.K
    model, ncpu = host_cpu()
    base_line = dict(value=round(tokens / t_total, 2), unit="tokens/s", cores=1, kind="oracle",
                     sample=f"{n_req} request(s) of {w.name} (K={w.K}, V={w.V}, r={w.r}), full "
                            f"draft of K tokens + verification of the scheduled prefix each, T>0 "
                            f"requests first; {t_total:.2f} s on one thread of {model} ({ncpu} "
                            f"logical CPUs); requests are independent, so the rate does not "
                            f"depend on B")
    parity = dict(requests=n_req, bit_exact=matched, near_ties=near,
                  rule="tokens, accepted length and next token equal, or an oracle near-tie "
                       "(< 1e-5)")
    return base_line, parity


def markov_vs_parallel(d, inp, seed, reps=10):
    """Draft-call time of the sequential Markov head against parallel drafting
    (every position from its own base logits, one pass) at K = 4 and K = 16 on
    the benchmark's requests and vocabulary."""
    import torch

    out = {}
    for K in (4, 16):
        base = inp["base"][:, :K].contiguous()
        res = {}
        for mode, A, W in (("markov", inp["A"], inp["W"]), ("parallel", None, None)):
            def call():
                d.dspark_draft_sample(base, A, W, inp["prev"], inp["temp"], seed)
            for _ in range(2):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            res[mode] = e0.elapsed_time(e1) / reps
        out[f"K={K}"] = {"markov_ms": round(res["markov"], 4),
                         "parallel_ms": round(res["parallel"], 4),
                         "markov_over_parallel": round(res["markov"] / res["parallel"], 3)}
    out["markov_K16_over_K4"] = round(out["K=16"]["markov_ms"] / out["K=4"]["markov_ms"], 3)
    out["parallel_K16_over_K4"] = round(out["K=16"]["parallel_ms"] / out["K=4"]["parallel_ms"], 3)
    return out


def gemm_latency_curve(dev, n_min, n_max, step=64, hidden=2560, inner=9728, reps=10):
    """Latency (ms) of one bf16 GEMM [N, hidden] x [hidden, inner] for N = n_min,
    n_min + step, ..., n_max: the shape of a 4B-class target model's MLP
    up-projection, a stand-in for the step latency of the target batch.  The
    library's tiling makes it a stair-step function of N."""
    import torch

    g = torch.Generator(device=dev).manual_seed(5)
    w = torch.randn((hidden, inner), generator=g, device=dev).to(torch.bfloat16)
    x = torch.randn((n_max, hidden), generator=g, device=dev).to(torch.bfloat16)
    ns, lat = [], []
    for n in range(n_min, n_max + 1, step):
        xn = x[:n]
        for _ in range(3):
            torch.matmul(xn, w)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(xn, w)
        e1.record()
        torch.cuda.synchronize()
        ns.append(float(n))
        lat.append(e0.elapsed_time(e1) / reps)
    return ns, lat


def objective(B, surv_sel_sum, n_tokens, ns, lat):
    """f(N) = (B + sum of selected S) / tau(N), tau piecewise linear in the
    curve points and flat outside them."""
    import numpy as np

    tau = float(np.interp(n_tokens, ns, lat))
    return (B + surv_sel_sum) / tau


def global_best(B, S, D, ns, lat):
    """max over n = 0..D of f(B + n) taking the n largest survival values: the
    global search over N the greedy early stop is compared with."""
    import numpy as np

    s = np.sort(S[S > 0].astype(np.float64))[::-1][:D]
    pre = np.concatenate([[0.0], np.cumsum(s)])
    n = np.arange(len(pre))
    f = (B + pre) / np.interp(B + n, ns, lat)
    i = int(np.argmax(f))
    return float(f[i]), int(B + i)


def sps_curve(d, inputs, dev, steps=12):
    """Next row 2: a measured stair-step curve in the confidence scheduler.
    Greedy early stop (the schedule kernel) against a global search over N on
    the confidence-scheduled workload, and the asynchronous variant whose
    budget comes from the confidences two steps back while the selection uses
    the current ones."""
    import numpy as np
    import torch

    w = inputs.WORKLOADS["conf_sched"]
    B, K, budget = w.B, w.K, w.budget
    D = max(0, budget - B)
    # the scheduler sees N in [B, budget]: 49 points at a step of 64 tokens
    ns, lat = gemm_latency_curve(dev, B, budget)
    jumps = [(int(ns[i]), round(lat[i] / lat[i - 1], 3)) for i in range(1, len(lat))
             if lat[i] > 1.15 * lat[i - 1]]

    def greedy(conf):
        L, _, S = d.dspark_schedule(conf, budget, ns, lat)
        torch.cuda.synchronize()
        L, S = L.cpu().numpy(), S.cpu().numpy()
        sel = sum(float(S[b, :L[b]].sum()) for b in range(B))
        n = B + int(L.sum())
        return L, S, n, objective(B, sel, n, ns, lat)

    confs = [inputs.make_confidence(w, dev, seed=100 + t)[0] for t in range(steps)]
    rows = []
    for t, conf in enumerate(confs):
        L, S, n_g, f_g = greedy(conf)
        f_star, n_star = global_best(B, S, D, ns, lat)
        row = {"n_greedy": n_g, "f_greedy": f_g, "n_global": n_star, "f_global": f_star}
        if t >= 2:
            # budget from the confidences of step t - 2, selection with the current ones
            _, _, n_lag, _ = greedy(confs[t - 2])
            Ll, _, Sl = d.dspark_schedule(conf, n_lag)
            torch.cuda.synchronize()
            Ll, Sl = Ll.cpu().numpy(), Sl.cpu().numpy()
            sel = sum(float(Sl[b, :Ll[b]].sum()) for b in range(B))
            row["n_lag"] = B + int(Ll.sum())
            row["f_lag"] = objective(B, sel, row["n_lag"], ns, lat)
        rows.append(row)
    lag = [r["f_lag"] / r["f_greedy"] for r in rows if "f_lag" in r]
    return {
        "curve": {"gemm": "bf16 [N, 2560] x [2560, 9728]", "n": [int(ns[0]), int(ns[-1])],
                  "points": len(ns),
                  "step": int(ns[1] - ns[0]), "ms_at_budget": round(float(np.interp(budget, ns, lat)), 4),
                  "jumps_over_15pct": jumps[:12]},
        "workload": f"conf_sched (B={B}, K={K}, budget {budget} tokens), {steps} steps of fresh "
                    f"confidences",
        "greedy_over_global": round(float(np.mean([r["f_greedy"] / r["f_global"] for r in rows])), 4),
        "n_greedy_mean": round(float(np.mean([r["n_greedy"] for r in rows])), 1),
        "n_global_mean": round(float(np.mean([r["n_global"] for r in rows])), 1),
        "lagged_over_greedy": round(float(np.mean(lag)), 4),
        "n_lag_mean": round(float(np.mean([r["n_lag"] for r in rows if "n_lag" in r])), 1),
    }


def ece(conf, label, bins=15):
    """Expected calibration error: over equal-width confidence bins, the
    sample-weighted mean of |mean label - mean confidence|."""
    import numpy as np

    c = np.asarray(conf, np.float64)
    y = np.asarray(label, np.float64)
    if c.size == 0:
        return 0.0
    idx = np.minimum((c * bins).astype(np.int64), bins - 1)
    err = 0.0
    for j in range(bins):
        m = idx == j
        if m.any():
            err += m.sum() * abs(y[m].mean() - c[m].mean())
    return float(err / c.size)


def sts_fit(c_raw, label, reached, lo=0.05, hi=20.0, min_samples=200):
    """Sequential temperature scaling: for positions k = 1..K in order, the
    temperature tau_k that minimises the Bernoulli log-loss of position k's
    acceptance labels over the samples that reached k (every earlier token
    accepted), with calibrated confidence sigmoid(logit(c_raw) / tau_k).  A
    position reached by fewer than min_samples samples keeps the temperature
    of the position before it (1 for the first)."""
    import numpy as np
    from scipy.optimize import minimize_scalar

    eps = 1e-6
    taus = []
    for k in range(c_raw.shape[1]):
        m = reached[:, k]
        if m.sum() < min_samples:
            taus.append(taus[-1] if taus else 1.0)
            continue
        c = np.clip(c_raw[m, k].astype(np.float64), eps, 1 - eps)
        x = np.log(c) - np.log1p(-c)
        y = label[m, k].astype(np.float64)

        def nll(lt):
            q = np.clip(1.0 / (1.0 + np.exp(-x / np.exp(lt))), eps, 1 - eps)
            return -np.mean(y * np.log(q) + (1 - y) * np.log1p(-q))

        res = minimize_scalar(nll, bounds=(np.log(lo), np.log(hi)), method="bounded")
        taus.append(float(np.exp(res.x)))
    return taus


def sts_apply(c_raw, taus):
    import numpy as np

    c = np.clip(c_raw.astype(np.float64), 1e-6, 1 - 1e-6)
    x = np.log(c) - np.log1p(-c)
    return 1.0 / (1.0 + np.exp(-x / np.asarray(taus)[None, :]))


def calibration(d, inp, w, dev, seeds=16, over=2.0):
    """Next row 3: confidence calibration on synthetic labels.  The synthetic
    confidence head predicts, for each drafted position, the exact conditional
    acceptance probability alpha_k = sum_v min(p_t, p_d) of the drafted prefix,
    made over-confident as sigmoid(over * logit(alpha_k)); the labels are the
    acceptance outcomes of dspark_verify (position k is labelled when every
    earlier token was accepted).  Sequential temperature scaling is fitted on
    half of the draws and the expected calibration error is measured on the
    other half."""
    import numpy as np
    import torch

    B, K, V = w.B, w.K, w.V
    sampled = (inp["temp"] > 0).cpu().numpy()
    tsafe = torch.where(inp["temp"] > 0, inp["temp"], torch.ones_like(inp["temp"]))
    it = (1.0 / tsafe).view(B, 1, 1)
    target = inp["target"]
    pt = torch.softmax(target[:, :K].float() * it, dim=-1)
    offs = torch.arange(B, dtype=torch.int64, device=dev) * (K + 1)
    Wf = inp["W"].float()
    craw, lab, rch = [], [], []
    for s in range(seeds):
        tok, logp, lse = d.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"],
                                               inp["temp"], 7000 + s)
        prevs = torch.cat([inp["prev"].view(B, 1), tok[:, :-1]], dim=1).long()
        alpha = torch.empty((B, K), device=dev)
        for k in range(K):
            bias = inp["A"][prevs[:, k]].float() @ Wf
            pd = torch.softmax((inp["base"][:, k].float() + bias) * it.view(B, 1), dim=-1)
            alpha[:, k] = torch.minimum(pd, pt[:, k]).sum(-1)
        acc, _, _, _ = d.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"],
                                       inp["W"], target.reshape(-1, V), offs, inp["temp"],
                                       9000 + s)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()[sampled]
        al = alpha.clamp(1e-6, 1 - 1e-6).cpu().numpy()[sampled]
        kk = np.arange(K)[None, :]
        lab.append((kk < a[:, None]).astype(np.float64))
        rch.append(kk <= a[:, None])
        lg = np.log(al) - np.log1p(-al)
        craw.append(1.0 / (1.0 + np.exp(-over * lg)))
    half = seeds // 2
    cf, yf, rf = (np.concatenate(x[:half]) for x in (craw, lab, rch))
    ce, ye, re_ = (np.concatenate(x[half:]) for x in (craw, lab, rch))
    taus = sts_fit(cf, yf, rf)
    cc = sts_apply(ce, taus)
    return {
        "head": f"synthetic: sigmoid({over} logit(alpha_k)), alpha_k = sum_v min(p_t, p_d) of the "
                f"drafted prefix; labels from dspark_verify",
        "requests": int(sampled.sum()), "draws": seeds, "fit_draws": half,
        "labelled_positions_eval": int(re_.sum()),
        "tau": [round(t, 3) for t in taus],
        "ece_raw": round(ece(ce[re_], ye[re_]), 4),
        "ece_sts": round(ece(cc[re_], ye[re_]), 4),
        "ece_raw_first4": [round(ece(ce[re_[:, k], k], ye[re_[:, k], k]), 4) for k in range(4)],
        "ece_sts_first4": [round(ece(cc[re_[:, k], k], ye[re_[:, k], k]), 4) for k in range(4)],
    }


def prepare(d, inputs, torch, w, dev, seed):
    """Inputs, outputs and workspaces of one workload, laid out before any
    timing, and the step that runs draft -> schedule -> verify on them."""
    inp = inputs.make_inputs(w, dev, seed=1, with_target=not w.ragged)
    conf, _ = inputs.make_confidence(w, dev, seed=1)
    B, K, V, r = w.B, w.K, w.V, w.r
    budget = w.budget if w.budget else B * (K + 1)
    cn, ct = w.curve()

    # outputs and workspaces allocated once, outside the timed region
    tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    logp = torch.empty((B, K), dtype=torch.float32, device=dev)
    lse = torch.empty((B, K), dtype=torch.float32, device=dev)
    L = torch.empty(B, dtype=torch.int32, device=dev)
    offs = torch.empty(B + 1, dtype=torch.int64, device=dev)
    surv = torch.empty((B, K), dtype=torch.float32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    ws_d = torch.empty(d.dspark_draft_workspace_bytes(B, K, V, r), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(256, d.dspark_schedule_workspace_bytes(B, K)), dtype=torch.uint8,
                       device=dev)
    ws_v = torch.empty(d.dspark_verify_workspace_bytes(B, K, V, r), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # The schedule depends on the confidences alone, so one call before timing
    # lays out the verify rows: ragged workloads get target rows for the
    # scheduled prefixes only, at the schedule's row offsets; dense ones read
    # the [B, K+1, V] tensor at offsets b (K+1) with the scheduled lengths.
    d.dspark_schedule(conf, budget, cn, ct, lengths=L, row_offsets=offs, survival=surv,
                      workspace=ws_s)
    torch.cuda.synchronize()
    if w.ragged:
        target = inputs.ragged_target(w, inp["base"], L, offs, dev, seed=1)
        vofs = offs
    else:
        target = inp["target"].reshape(-1, V)
        vofs = inputs.dense_offsets(B, K, dev)
    torch.cuda.synchronize()

    def step(events=None):
        if events:
            events[0].record(stream)
        d.dspark_draft_sample(inp["base"], inp["A"], inp["W"], inp["prev"], inp["temp"], seed,
                              draft_tokens=tok, draft_logp=logp, draft_lse=lse, workspace=ws_d)
        if events:
            events[1].record(stream)
        d.dspark_schedule(conf, budget, cn, ct, lengths=L, row_offsets=offs, survival=surv,
                          workspace=ws_s)
        if events:
            events[2].record(stream)
        d.dspark_verify(tok, inp["prev"], logp, lse, inp["base"], inp["A"], inp["W"], target,
                        vofs, inp["temp"], seed, L, accepted=acc, next_token=nxt,
                        row_outputs=False, workspace=ws_v)
        if events:
            events[3].record(stream)

    return SimpleNamespace(inp=inp, conf=conf, B=B, K=K, V=V, r=r, budget=budget, tok=tok,
                           logp=logp, lse=lse, L=L, offs=offs, acc=acc, nxt=nxt, target=target,
                           vofs=vofs, stream=stream, step=step)


def quick_workload(d, inputs, torch, name, dev, seed, steps=5, warmup=1):
    """A short timed run of another workload (its own inputs at full size):
    tokens/s over `steps` steps after `warmup`, and the phases of one more
    step bracketed with events."""
    w = inputs.WORKLOADS[name]
    st = prepare(d, inputs, torch, w, dev, seed)
    for _ in range(warmup):
        st.step()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st.stream)
    for _ in range(steps):
        st.step()
    t1.record(st.stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    st.step(ev)
    torch.cuda.synchronize()
    out = {"B": w.B, "K": w.K, "V": w.V, "budget_tokens": st.budget,
           "tokens_per_s": round(w.B * w.K / (ms_step / 1e3), 1), "ms_per_step": round(ms_step, 4),
           "steps": steps, "warmup": warmup,
           "phases_ms": {"draft": round(ev[0].elapsed_time(ev[1]), 4),
                         "schedule": round(ev[1].elapsed_time(ev[2]), 4),
                         "verify": round(ev[2].elapsed_time(ev[3]), 4)},
           "verified_tokens_per_step": int(st.L.sum())}
    del st
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): requests are "
              "independent, so more GPUs would each run this same path on their own share of "
              "the batch, and no multi-GPU figure is produced", file=sys.stderr)
        sys.exit(2)
    import torch

    import draft_sampling_verification_04_amd as d
    from draft_sampling_verification_04_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    d.lib()
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    seed = 20260627
    st = prepare(d, inputs, torch, w, dev, seed)
    inp, conf, B, K, V, r, budget = st.inp, st.conf, st.B, st.K, st.V, st.r, st.budget
    tok, logp, lse, L, offs, acc, nxt = st.tok, st.logp, st.lse, st.L, st.offs, st.acc, st.nxt
    target, vofs, stream, step = st.target, st.vofs, st.stream, st.step

    if args.copy_probe_mib > 0:
        # reference kernel for counter scaling: reads and writes exactly N MiB
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region.  Events perturb what they time (each one recorded between
    # two dependent kernels widens the gap between them), so only the last
    # `inst` steps are instrumented: their phases are bracketed with events, and
    # the library brackets each launch of the dominant kernel (the draft strip
    # kernel, K launches per step) with HIP events on the stream it is
    # launched on.  The other steps run as they would in production.
    inst = min(args.steps, 2)
    phase_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                    for _ in range(inst)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        j = i - (args.steps - inst)
        if j == 0:
            d.dspark_profile_begin(("draft_strip",), max_launches=K * inst)
        step(phase_events[j] if j >= 0 else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    prof = d.dspark_profile_end()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    draft_ms = sum(e[0].elapsed_time(e[1]) for e in phase_events) / inst
    sched_ms = sum(e[1].elapsed_time(e[2]) for e in phase_events) / inst
    verify_ms = sum(e[2].elapsed_time(e[3]) for e in phase_events) / inst
    strip_ms, _, strip_timed = prof["draft_strip"]
    strip_avg_s = strip_ms / max(strip_timed, 1) / 1e3

    # One more (untimed) pass over a few steps with every kernel bracketed,
    # for the per-kernel table.
    d.dspark_profile_begin(d.KERNELS, max_launches=64 * max(1, min(args.steps, 5)))
    for _ in range(max(1, min(args.steps, 5))):
        step()
    torch.cuda.synchronize()
    per_kernel = d.dspark_profile_end()

    verified = int(L.sum())
    emitted = int(acc.sum()) + B
    rows_read = target_rows_read(L.cpu().tolist(), acc.cpu().tolist(), K)
    tokens_per_s = B * K / (ms_step / 1e3)
    prof_steps = max(1, min(args.steps, 5))

    es = 2 if w.dtype == torch.bfloat16 else 4
    # Algorithmic bytes (what the method must read at least once):
    # draft call: every base logit plus W once (the K steps share it) plus the
    # gathered A rows; per launch of the draft strip kernel (one draft step)
    # that is a K-th of the base-plus-W figure.
    draft_bytes = es * (B * K * V + r * V + K * B * r)
    strip_bytes = draft_bytes / K
    reread_bytes = es * (B * V + r * V + B * r)
    strip_flops = 2.0 * B * r * V
    achieved_gbs = strip_bytes / strip_avg_s / 1e9
    stored = stored_counters()
    traffic = stored["traffic_bytes_per_launch"] if stored else None
    # verify rows: every target row read under the early-exit schedule, once
    rows_ms, _, rows_timed = per_kernel["verify_rows"]
    rows_bytes = es * rows_read * V
    # residual strip: a sampled rejection reads its recomputed draft row and
    # its target row, a sampled full acceptance its bonus row; W once
    sampled = inp["temp"] > 0
    n_rej = int(((acc < L) & sampled).sum())
    n_bonus = int(((acc >= L) & sampled).sum())
    res_ms, _, res_timed = per_kernel["residual_strip"]
    res_bytes = es * ((2 * n_rej + n_bonus) * V + r * V + (n_rej + n_bonus) * r)
    step_bytes = draft_bytes + rows_bytes + res_bytes

    def gbs(nbytes, ms, n):
        """GB/s of nbytes moved per unit, at ms total over n units."""
        return round(nbytes / (ms / max(n, 1) / 1e3) / 1e9, 1) if n else None

    def frac(g):
        return round(g / HBM_PEAK_GBS, 4) if g is not None else None

    kernels = {}
    for k, (ms, n, nt) in per_kernel.items():
        kernels[k] = {"launches_per_step": round(n / prof_steps, 2),
                      "avg_launch_us": round(1e3 * ms / nt, 2) if nt else None}
    g_strip = gbs(strip_bytes, *per_kernel["draft_strip"][::2])
    kernels["draft_strip"].update(
        bytes_per_launch=int(strip_bytes), hbm_gbs=g_strip, hbm_frac=frac(g_strip),
        mfma_tflops=round(strip_flops / (per_kernel["draft_strip"][0] /
                                         max(per_kernel["draft_strip"][2], 1) / 1e3) / 1e12, 1))
    g_rows = gbs(rows_bytes, rows_ms, prof_steps)
    kernels["verify_rows"].update(bytes_per_step=rows_bytes, hbm_gbs=g_rows, hbm_frac=frac(g_rows),
                                  target_rows_read_per_step=rows_read,
                                  target_rows_scheduled_per_step=verified + B)
    g_res = gbs(res_bytes, res_ms, prof_steps)
    kernels["residual_strip"].update(bytes_per_step=res_bytes, hbm_gbs=g_res, hbm_frac=frac(g_res),
                                     sampled_rejections=n_rej, sampled_bonus_rows=n_bonus)
    g_step = step_bytes / (ms_step / 1e3) / 1e9

    model, ncpu = host_cpu()
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "K": K, "V": V, "r": r,
                   "temperatures": list(w.temps), "budget_tokens": budget,
                   "target_rows": "ragged, scheduled prefixes only" if w.ragged
                   else "dense [B, K+1, V] at offsets b(K+1)",
                   "verify": ("every drafted token" if not w.budget else "scheduled prefixes")
                             + "; target rows read up to each request's first rejection "
                               "(position launches "
                             + ", ".join(f"{a}-{b}" for a, b in verify_position_launches(K))
                             + ")",
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "draft_strip_mfma_rk<8,16>" if r == 256 else "draft_strip_mfma",
            "algorithmic_bytes_per_launch": int(strip_bytes),
            "bytes_rule": "(base logits + W once + gathered A rows of one draft call) / K",
            "reread_bytes_per_launch": int(reread_bytes),
            "reread_frac": round(reread_bytes / strip_avg_s / 1e9 / HBM_PEAK_GBS, 4),
            "reread_rule": "base slice + all of W + gathered A rows: what one launch must read, "
                           "since step k's bias needs x_(k-1)",
            "avg_launch_us": round(strip_avg_s * 1e6, 2),
            "launches_timed": strip_timed,
            "timed_steps": f"last {inst} of {args.steps}",
            "mfma_tflops": round(strip_flops / strip_avg_s / 1e12, 1),
            "mfma_frac": round(strip_flops / strip_avg_s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "alu": alu_view(stored, strip_avg_s),
            "step": {"bytes": int(step_bytes), "achieved": round(g_step, 1),
                     "frac": round(g_step / HBM_PEAK_GBS, 4),
                     "bytes_rule": "draft call + verify rows read + residual/bonus rows"},
        },
        "phases_ms": {"draft": round(draft_ms, 4), "schedule": round(sched_ms, 4),
                      "verify": round(verify_ms, 4)},
        "kernels": kernels,
        "emitted_tokens_per_s": round(emitted / (ms_step / 1e3), 1),
        "vocab_logits_per_s": round((B * K * V + rows_read * V) / (ms_step / 1e3), 1),
        "host_cpu": f"{model} x{ncpu}",
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["oracle_parity"] = cpu_baseline(
            w, inp, seed, args.cpu_requests, target, vofs, L, (tok, acc, nxt))
    # The other measurements run after the headline one, outside its timed
    # region: the cost of the sequential head against parallel drafting, a
    # measured stair-step latency curve in the scheduler, calibration of a
    # synthetic confidence head, and short runs of the budgeted workloads.
    extras = not args.no_extras
    if args.markov_vs_parallel or extras:
        out["markov_vs_parallel"] = markov_vs_parallel(d, inp, seed)
    if args.sps_curve or extras:
        out["sps_curve"] = sps_curve(d, inputs, dev)
    if args.calibration or (extras and not w.ragged):
        if w.ragged:
            raise SystemExit("--calibration needs a workload with dense target rows")
        out["calibration"] = calibration(d, inp, w, dev)
    if extras:
        out["other_workloads"] = {
            name: quick_workload(d, inputs, torch, name, dev, seed)
            for name in ("qwen3_4b", "conf_sched", "high_conc") if name != w.name}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
