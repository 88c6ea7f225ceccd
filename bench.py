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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_draft")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=24)
    return ap.parse_args()


def cpu_baseline(w, inp, seed, n_req):
    """Time the oracle (single-threaded C) on n_req requests of the same
    workload: full draft of K tokens plus full verification."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import numpy as np
    import oracle as orc

    A = inp["A"].float().cpu().numpy()
    W = inp["W"].float().cpu().numpy()
    prev = inp["prev"].cpu().numpy()
    temp = inp["temp"].cpu().numpy()
    # sample requests with T > 0 (the expensive, sampled case) first
    order = sorted(range(w.B), key=lambda b: (temp[b] == 0.0, b))[:n_req]
    t_total = 0.0
    for b in order:
        base = inp["base"][b].float().cpu().numpy()
        rows = inp["target"][b].float().cpu().numpy()
        t0 = time.perf_counter()
        tok, _, _, _ = orc.draft_request(base, A, W, int(prev[b]), float(temp[b]), seed, b)
        orc.verify_request(tok, int(prev[b]), base, A, W, rows, w.K, float(temp[b]), seed, b)
        t_total += time.perf_counter() - t0
    tokens = n_req * w.K
    return dict(value=tokens / t_total, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n_req} request(s) of {w.name} (K={w.K}, V={w.V}, r={w.r}), full draft + "
                       f"verify of K tokens, T>0 first; {t_total:.2f} s; requests are independent, "
                       f"so the rate scales linearly with B")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over requests without communication, see DESIGN.md",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import draft_sampling_verification_04_amd as d
    from draft_sampling_verification_04_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    d.lib()
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    seed = 20260627
    inp = inputs.make_inputs(w, dev, seed=1)
    conf, _ = inputs.make_confidence(w, dev, seed=1)
    B, K, V, r = w.B, w.K, w.V, w.r
    budget = w.budget if w.budget else B * (K + 1)
    cn, ct = w.curve()
    target = inp["target"].reshape(-1, V)

    # outputs and workspaces allocated once, outside the timed region
    tok = torch.empty((B, K), dtype=torch.int32, device=dev)
    logp = torch.empty((B, K), dtype=torch.float32, device=dev)
    lse = torch.empty((B, K), dtype=torch.float32, device=dev)
    L = torch.empty(B, dtype=torch.int32, device=dev)
    offs = torch.empty(B + 1, dtype=torch.int64, device=dev)
    surv = torch.empty((B, K), dtype=torch.float32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    rows = target.shape[0]
    rl = torch.empty(rows, dtype=torch.float32, device=dev)
    rr = torch.empty(rows, dtype=torch.float32, device=dev)
    ws_d = torch.empty(d.dspark_draft_workspace_bytes(B, K, V, r), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(256, d.dspark_schedule_workspace_bytes(B, K)), dtype=torch.uint8,
                       device=dev)
    ws_v = torch.empty(d.dspark_verify_workspace_bytes(B, K, V, r), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

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
                        offs, inp["temp"], seed, L, accepted=acc, next_token=nxt, row_lse_t=rl,
                        row_logratio=rr, workspace=ws_v)
        if events:
            events[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    phase_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                    for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(phase_events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    draft_ms = sum(e[0].elapsed_time(e[1]) for e in phase_events) / args.steps
    sched_ms = sum(e[1].elapsed_time(e[2]) for e in phase_events) / args.steps
    verify_ms = sum(e[2].elapsed_time(e[3]) for e in phase_events) / args.steps
    verified = int(L.sum())
    emitted = int(acc.sum()) + B
    tokens_per_s = B * K / (ms_step / 1e3)

    es = 2 if w.dtype == torch.bfloat16 else 4
    draft_bytes = es * (B * K * V + r * V)  # base once + W once
    verify_bytes = es * ((verified + B) * V + r * V)
    draft_flops = 2.0 * B * r * V * K
    out = {
        "metric": "draft+verify tokens/s at B=256,K=16,V=151936",
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
                   "parallelism": "single GPU"},
        "phases_ms": {"draft": round(draft_ms, 4), "schedule": round(sched_ms, 4),
                      "verify": round(verify_ms, 4)},
        "emitted_tokens_per_s": round(emitted / (ms_step / 1e3), 1),
        "vocab_logits_per_s": round((B * K * V + (verified + B) * V) / (ms_step / 1e3), 1),
        "draft_call_hbm_gbs": round(draft_bytes / (draft_ms / 1e3) / 1e9, 1),
        "verify_call_hbm_gbs": round(verify_bytes / (verify_ms / 1e3) / 1e9, 1),
        "draft_call_tflops": round(draft_flops / (draft_ms / 1e3) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, seed, args.cpu_requests)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
