"""Seeded synthetic workloads (random inputs only; none of the method's arithmetic).

The DSpark write-ups measure on Qwen3 targets, nine benchmark datasets and
production traffic, none of which is available; these generators stand in
with the shapes and value distributions of the five named workloads:

  tiny        B=4,    K=4,  V=1024,   r=16,  fp32, base N(0,2), factors N(0,0.1),
              target = base + N(0,0.5), T=1
  qwen3_4b    B=64,   K=8,  V=151936, r=256, bf16, base N(0,3) with a +8 spike on
              one uniform token per row, factors N(0,0.05), target = base + N(0,1), T=1
  long_draft  B=256,  K=16, V=151936, r=256, bf16, qwen3_4b distributions,
              T uniform in {0, 0.7, 1}, target noise sd 0.5 -> 2.0 along the rows
  conf_sched  B=1024, K=16, V=151936, r=256, bf16, qwen3_4b distributions,
              confidences Beta(mu*20, (1-mu)*20) with mu falling linearly from 0.9
              to 0.3 / 0.6 / 0.8 for a 40/30/30 chat/math/code mix, budget 4096,
              latency curve flat to 4096 tokens then slope 1.5 per 4096; target
              rows generated for the scheduled prefixes only (ragged)
  high_conc   B=2048, K=16, V=131072, r=256, bf16, long_draft distributions,
              mixed T, budget 8192 (same curve shape), dense target rows [B, K+1, V]
              read at offsets b (K+1) with the scheduled lengths

The target logits of row j are the backbone logits of an extended draft block
(K+1 rows) plus Gaussian noise; the transition bias is not part of them.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    r: int
    dtype: torch.dtype
    base_sd: float
    spike: float
    factor_sd: float
    noise_lo: float
    noise_hi: float
    temps: tuple
    budget: int = 0  # 0: verify every drafted token
    ragged: bool = False  # target rows for the scheduled prefixes only (else dense [B, K+1, V])

    def curve(self):
        """Step-latency curve: flat up to `budget` tokens, then +1.5x per `budget`."""
        if not self.budget:
            return None, None
        return [float(self.budget), 2.0 * self.budget], [1.0, 2.5]


WORKLOADS = {
    "tiny": Workload("tiny", 4, 4, 1024, 16, torch.float32, 2.0, 0.0, 0.1, 0.5, 0.5, (1.0,)),
    "qwen3_4b": Workload("qwen3_4b", 64, 8, 151936, 256, torch.bfloat16, 3.0, 8.0, 0.05, 1.0,
                         1.0, (1.0,)),
    "long_draft": Workload("long_draft", 256, 16, 151936, 256, torch.bfloat16, 3.0, 8.0, 0.05,
                           0.5, 2.0, (0.0, 0.7, 1.0)),
    "conf_sched": Workload("conf_sched", 1024, 16, 151936, 256, torch.bfloat16, 3.0, 8.0, 0.05,
                           1.0, 1.0, (1.0,), budget=4096, ragged=True),
    "high_conc": Workload("high_conc", 2048, 16, 131072, 256, torch.bfloat16, 3.0, 8.0, 0.05,
                          0.5, 2.0, (0.0, 0.7, 1.0), budget=8192),
}

TASK_MIX = (("chat", 0.4, 0.3), ("math", 0.3, 0.6), ("code", 0.3, 0.8))


def resized(w: Workload, **kw) -> Workload:
    return dataclasses.replace(w, **kw)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_inputs(w: Workload, device="cuda", seed=0, with_target=True, chunk=32):
    """Draft-side inputs and (optionally) dense target rows [B, K+1, V]."""
    g = _gen(device, seed)
    B, K, V, r = w.B, w.K, w.V, w.r
    A = (torch.randn((V, r), generator=g, device=device) * w.factor_sd).to(w.dtype)
    W = (torch.randn((r, V), generator=g, device=device) * w.factor_sd).to(w.dtype)
    prev = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int32)
    ti = torch.randint(0, len(w.temps), (B,), generator=g, device=device)
    temp = torch.tensor(w.temps, dtype=torch.float32, device=device)[ti].contiguous()
    base = torch.empty((B, K, V), dtype=w.dtype, device=device)
    target = torch.empty((B, K + 1, V), dtype=w.dtype, device=device) if with_target else None
    sd = torch.tensor([w.noise_lo + (w.noise_hi - w.noise_lo) * j / K for j in range(K + 1)],
                      dtype=torch.float32, device=device).view(1, K + 1, 1)
    for b0 in range(0, B, chunk):
        nb = min(chunk, B - b0)
        ext = torch.randn((nb, K + 1, V), generator=g, device=device) * w.base_sd
        if w.spike:
            hot = torch.randint(0, V, (nb, K + 1, 1), generator=g, device=device)
            ext.scatter_add_(2, hot, torch.full((nb, K + 1, 1), w.spike, device=device))
        base[b0:b0 + nb] = ext[:, :K].to(w.dtype)
        if with_target:
            noise = torch.randn((nb, K + 1, V), generator=g, device=device) * sd
            target[b0:b0 + nb] = (ext + noise).to(w.dtype)
        del ext
    return dict(base=base, A=A, W=W, prev=prev, temp=temp, target=target)


def make_confidence(w: Workload, device="cuda", seed=0, kappa=20.0):
    """c[b, k] ~ Beta(mu_k kappa, (1 - mu_k) kappa); mu falls linearly from 0.9 at
    k = 1 to the task's end value at k = K; tasks drawn by the 40/30/30 mix."""
    g = _gen(device, seed + 7919)
    B, K = w.B, w.K
    probs = torch.tensor([m[1] for m in TASK_MIX], device=device)
    task = torch.multinomial(probs, B, replacement=True, generator=g)
    ends = torch.tensor([m[2] for m in TASK_MIX], dtype=torch.float64, device=device)[task]
    frac = torch.arange(K, dtype=torch.float64, device=device) / max(K - 1, 1)
    mu = 0.9 + (ends.view(B, 1) - 0.9) * frac.view(1, K)
    # Beta via two Gamma draws (torch.distributions takes no generator)
    a = (mu * kappa).float()
    bb = ((1.0 - mu) * kappa).float()
    ga = torch._standard_gamma(a, generator=g)
    gb = torch._standard_gamma(bb, generator=g)
    conf = (ga / (ga + gb)).clamp(0.0, 1.0).contiguous()
    return conf, task


def ragged_target(w: Workload, base, lengths, row_offsets, device="cuda", seed=0):
    """Target rows for the scheduled prefixes only ([sum(L_b + 1), V])."""
    g = _gen(device, seed + 104729)
    B, K, V = w.B, w.K, w.V
    L = lengths.to("cpu").tolist()
    offs = row_offsets.to("cpu").tolist()
    rows = int(offs[B])
    out = torch.empty((rows, V), dtype=w.dtype, device=device)
    for b in range(B):
        n = L[b] + 1
        j = torch.arange(n, device=device, dtype=torch.float32)
        sd = (w.noise_lo + (w.noise_hi - w.noise_lo) * j / K).view(n, 1)
        src = torch.empty((n, V), dtype=torch.float32, device=device)
        m = min(n, K)
        src[:m] = base[b, :m].float()
        if n > K:  # bonus row past the drafted block: a fresh backbone row
            src[K:] = torch.randn((n - K, V), generator=g, device=device) * w.base_sd
        noise = torch.randn((n, V), generator=g, device=device) * sd
        out[offs[b]:offs[b] + n] = (src + noise).to(w.dtype)
    return out


def dense_offsets(B, K, device="cuda"):
    return (torch.arange(B, dtype=torch.int64, device=device) * (K + 1)).contiguous()


def gib(n_bytes) -> float:
    return n_bytes / float(1 << 30)


def approx_bytes(w: Workload) -> int:
    es = 2 if w.dtype == torch.bfloat16 else 4
    return es * (w.B * w.K * w.V + w.B * (w.K + 1) * w.V + 2 * w.V * w.r) + int(math.ceil(w.B))
