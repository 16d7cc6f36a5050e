"""Seeded synthetic workloads for the sparse-MoE FFN layer.

This module only draws random numbers: it holds none of the layer's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.  All
draws are fp32 from a torch CPU generator, then rounded to bf16 (round to
nearest even, torch's conversion) where the workload stores bf16.

Every tensor has its own generator stream, seeded with seed*1000 + a fixed
index (u 0, w_router 1, b_router 2, w_gate 3, w_up 4, w_down 5, ws_gate 6,
ws_up 7, ws_down 8, noise 9), so any subset can be drawn alone and comes out
the same.  Distributions: u ~ N(0, 1); weights ~ N(0, std)
with std = 1/sqrt(fan_in) unless the workload fixes it (the second argument
of N(.,.) is the standard deviation).
"""
import dataclasses
import math
from dataclasses import dataclass
from typing import Dict, Optional

import torch

GATINGS = ("softmax_topk", "topk_softmax")   # all-N softmax, unrenormalised | top-K then softmax
ACTS = ("swiglu", "relu")
DTYPES = ("f32", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    N: int
    K: int
    d_ff: int
    n_shared: int = 0
    d_ff_shared: int = 0
    capacity_factor: float = 0.0       # <= 0: no capacity limit
    noise_weight: float = 0.0
    gating: str = "topk_softmax"
    act: str = "swiglu"
    dtype: str = "bf16"
    seed: int = 0
    router_std: Optional[float] = None  # None: 1/sqrt(d)
    expert_std: Optional[float] = None  # None: 1/sqrt(fan_in)
    bias: str = "none"                  # none | hot2 | zipf
    hot_bias: float = 0.70              # hot2: bias added to two seeded experts
    zipf_s: float = 1.2                 # zipf: exponent of the load ranking
    noise: bool = False
    drop_order: str = "token"           # token | choice: priority under capacity

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def es(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 layer: top-2, softmax over the selected scores, SwiGLU
    "tiny_fp32": Workload("tiny_fp32", T=256, d=64, N=4, K=2, d_ff=128,
                          gating="topk_softmax", act="swiglu", dtype="f32", seed=1001),
    # Switch-style top-1 with capacity factor 1.25 and two hot experts
    "switch_top1": Workload("switch_top1", T=4096, d=768, N=8, K=1, d_ff=3072,
                            capacity_factor=1.25, gating="softmax_topk", act="relu",
                            dtype="bf16", seed=1002, bias="hot2"),
    # Mixtral-shaped: top-2, softmax over the selected scores, SwiGLU
    "mixtral": Workload("mixtral", T=8192, d=4096, N=8, K=2, d_ff=14336,
                        gating="topk_softmax", act="swiglu", dtype="bf16", seed=1003,
                        router_std=0.02, expert_std=0.02),
    # DeepSeekMoE-shaped: 64 fine-grained experts, top-6 of an all-64 softmax,
    # unrenormalised gates, two always-on shared experts
    "deepseekmoe": Workload("deepseekmoe", T=16384, d=2048, N=64, K=6, d_ff=1408,
                            n_shared=2, d_ff_shared=1408, gating="softmax_topk",
                            act="swiglu", dtype="bf16", seed=1004),
    # decode-sized, Zipf-skewed router bias, noisy top-8
    "decode_noisy": Workload("decode_noisy", T=128, d=4096, N=128, K=8, d_ff=1536,
                             noise_weight=1.0, gating="topk_softmax", act="swiglu",
                             dtype="bf16", seed=1005, bias="zipf", noise=True),
}

ORDER = ("tiny_fp32", "switch_top1", "mixtral", "deepseekmoe", "decode_noisy")

_CHUNK = 1 << 24   # draw big matrices in chunks of this many values


def _normal(g: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    """N(0, std) drawn in fp32 chunk by chunk, stored as `dtype`."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        flat[s:e] = torch.empty(e - s, dtype=torch.float32).normal_(0.0, std, generator=g).to(dtype)
    return out


def harmonic(n: int, s: float) -> float:
    """Generalised harmonic number H_{n,s} = sum_{r=1..n} r^-s."""
    return math.fsum(r ** -s for r in range(1, n + 1))


STREAMS = dict(u=0, w_router=1, b_router=2, w_gate=3, w_up=4, w_down=5, ws_gate=6, ws_up=7,
               ws_down=8, noise=9)
ROUTER = ("u", "w_router", "b_router", "noise")


def _gen(w: Workload, name: str) -> torch.Generator:
    return torch.Generator().manual_seed(w.seed * 1000 + STREAMS[name])


def generate(w: Workload, only=None) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of workload `w` as CPU tensors (weights row-major [out][in]).
    `only`: names to draw (default all); the others are None."""
    want = set(STREAMS) if only is None else set(only)
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, d, N, dff = w.T, w.d, w.N, w.d_ff
    x: Dict[str, Optional[torch.Tensor]] = {k: None for k in STREAMS}
    if "u" in want:
        x["u"] = _normal(_gen(w, "u"), (T, d), 1.0, et)
    if "w_router" in want:
        x["w_router"] = _normal(_gen(w, "w_router"), (N, d), w.router_std or 1.0 / math.sqrt(d),
                                torch.float32)
    if "b_router" in want and w.bias != "none":
        g = _gen(w, "b_router")
        if w.bias == "hot2":
            # two seeded experts get a positive bias so that they draw about
            # twice the mean load
            hot = torch.randperm(N, generator=g)[:2]
            b = torch.zeros(N, dtype=torch.float32)
            b[hot] = w.hot_bias
        elif w.bias == "zipf":
            # seeded ranking r_e (a permutation of 1..N); softmax(b) is the
            # Zipf pmf r^-s / H_{N,s}
            r = (torch.randperm(N, generator=g) + 1).to(torch.float64)
            b = (-w.zipf_s * torch.log(r) - math.log(harmonic(N, w.zipf_s))).to(torch.float32)
        else:
            raise ValueError(w.bias)
        x["b_router"] = b
    sd_in = w.expert_std or 1.0 / math.sqrt(d)
    sd_ff = w.expert_std or 1.0 / math.sqrt(dff)
    if "w_gate" in want:
        x["w_gate"] = _normal(_gen(w, "w_gate"), (N, dff, d), sd_in, et)
    if "w_up" in want and w.act == "swiglu":
        x["w_up"] = _normal(_gen(w, "w_up"), (N, dff, d), sd_in, et)
    if "w_down" in want:
        x["w_down"] = _normal(_gen(w, "w_down"), (N, d, dff), sd_ff, et)
    if w.n_shared > 0:
        ds = w.d_ff_shared
        sd_ffs = w.expert_std or 1.0 / math.sqrt(ds)
        if "ws_gate" in want:
            x["ws_gate"] = _normal(_gen(w, "ws_gate"), (w.n_shared, ds, d), sd_in, et)
        if "ws_up" in want and w.act == "swiglu":
            x["ws_up"] = _normal(_gen(w, "ws_up"), (w.n_shared, ds, d), sd_in, et)
        if "ws_down" in want:
            x["ws_down"] = _normal(_gen(w, "ws_down"), (w.n_shared, d, ds), sd_ffs, et)
    if "noise" in want and w.noise:
        x["noise"] = _normal(_gen(w, "noise"), (T, N), 1.0, torch.float32)
    return x


def random_topk(T: int, N: int, K: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """Seeded expert choices [T][K] int32: K distinct experts per token,
    drawn without replacement with weights (rank)^-skew (0: uniform)."""
    g = torch.Generator().manual_seed(seed)
    wts = torch.arange(1, N + 1, dtype=torch.float64) ** (-skew)
    wts = wts[torch.randperm(N, generator=g)]
    if T == 0:
        return torch.zeros((0, K), dtype=torch.int32)
    return torch.multinomial(wts.expand(T, N), K, replacement=False, generator=g).to(torch.int32)
