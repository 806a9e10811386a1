"""Seeded synthetic workloads for Top-K+phi decode (input generation only).

This module draws the inputs that both the HIP path and the CPU oracle consume:
KV caches, decode queries and the random feature-map parameters.  It contains
none of the method's arithmetic (no scores, no selection, no features, no
summaries): only random draws, the planting of needle keys, and the rounding of
stored K/V to their storage precision.

The five workloads follow the shapes of the Llama-3.2-1B/3B backbones that
"Residual-Mass Accounting for Partial-KV Decoding" evaluates (§5.1: 1B and 3B
Instruct; GQA 32/8 at head dim 64 and 24/8 at head dim 128), its 0.5-4 %
exact-support budgets (§5.2, Table 1) and its sink/tail anchor split (§3).
The pages evaluate on LongBench, RULER and BABILong; none of those are used
here.  Seeded Gaussian keys with a shared per-head offset (sink-like bias),
planted near-aligned "needle" keys (retrieval targets) and two query scales
(diffuse vs concentrated heads, §6) stand in for them.

Unit order: a unit is one (request, layer, kv head); units are ordered with the
request outermost, then the layer, then the kv head, so unit u uses parameter
set p = u % (layers * h_kv).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    layers: int
    h_q: int
    h_kv: int
    d: int
    L: int               # prefill length
    n_sink: int
    n_tail: int
    K: tuple             # retrieved tokens per query head (one or a sweep)
    m: int               # feature dimension of phi
    steps: int           # decode steps (generated tokens appended at L, L+1, ...)
    kv_dtype: str        # "f32" or "bf16"
    phi_dtype: str       # storage dtype of the stored phi(k) rows
    key_offset_norm: float
    q_scale_mode: str    # "one", "heads_half", "layers_alt"
    needle_mode: str     # "planted3" or "frac"
    seed: int
    desc: str = ""

    @property
    def G(self) -> int:
        return self.h_q // self.h_kv

    @property
    def U(self) -> int:
        return self.batch * self.layers * self.h_kv

    @property
    def P(self) -> int:
        return self.layers * self.h_kv

    @property
    def n_anchor(self) -> int:
        return self.n_sink + self.n_tail

    @property
    def L_mid(self) -> int:
        return self.L - self.n_sink - self.n_tail

    @property
    def T_cap(self) -> int:
        # single-step workloads decode against the prefill segment only
        return self.L + (self.steps if self.steps > 1 else 0)

    def n_gen(self, step: int) -> int:
        """Generated tokens visible at decode step `step` (0-based)."""
        return step + 1 if self.steps > 1 else 0

    @property
    def queries_per_step(self) -> int:
        return self.U * self.G

    def torch_kv_dtype(self):
        return torch.float32 if self.kv_dtype == "f32" else torch.bfloat16

    def torch_phi_dtype(self):
        return torch.float32 if self.phi_dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c0": Config("c0", 1, 1, 2, 1, 64, 1024, 4, 32, (10,), 64, 1, "f32", "f32", 0.0,
                 "one", "planted3", 0,
                 "tiny fp32 case: 2 query heads on 1 kv head, d=64, L=1024, K=10"),
    "c1": Config("c1", 1, 1, 32, 8, 64, 32768, 4, 64, (328,), 128, 1, "bf16", "bf16", 3.0,
                 "heads_half", "frac", 1,
                 "1B-shaped layer: GQA 32/8, d=64, 32K context, 1% budget (K=328)"),
    "c2": Config("c2", 1, 1, 24, 8, 128, 65536, 4, 64, (327, 655, 1310, 2621), 128, 1, "bf16",
                 "bf16", 3.0, "heads_half", "frac", 2,
                 "3B-shaped layer: GQA 24/8, d=128, 64K context, 0.5-4% budget sweep"),
    "c3": Config("c3", 16, 16, 32, 8, 64, 16384, 4, 64, (163,), 128, 8, "bf16", "bf16", 0.0,
                 "one", "frac", 3,
                 "1B-shaped stack: 16 requests x 16 layers, 16K context, 8 decode steps"),
    "c4": Config("c4", 4, 28, 24, 8, 128, 131072, 4, 64, (1310,), 128, 8, "bf16", "bf16", 3.0,
                 "layers_alt", "frac", 4,
                 "3B-shaped stack: 4 requests x 28 layers, 128K context, 1% budget"),
}


def query_scale(cfg: Config, unit: int) -> float:
    """Query scale of every query head in `unit` (diffuse 0.3 vs peaked 2.0)."""
    if cfg.q_scale_mode == "one":
        return 1.0
    h = unit % cfg.h_kv
    layer = (unit // cfg.h_kv) % cfg.layers
    if cfg.q_scale_mode == "heads_half":
        # query heads j = h*G + g; the first half of the query heads are diffuse
        return 0.3 if h * cfg.G < cfg.h_q // 2 else 2.0
    if cfg.q_scale_mode == "layers_alt":
        return 0.3 if layer % 2 == 0 else 2.0
    raise ValueError(cfg.q_scale_mode)


def n_needles(cfg: Config) -> int:
    if cfg.needle_mode == "planted3":
        return 3
    return int(round(0.001 * cfg.L))


@dataclasses.dataclass
class Inputs:
    cfg: Config
    k: torch.Tensor          # [U, T_cap, d] kv dtype
    v: torch.Tensor          # [U, T_cap, d] kv dtype
    q: torch.Tensor          # [steps, U, G, d] float32
    W: torch.Tensor          # [P, m, d] float32 (phi parameters, shared by phi_q and phi_k)
    b: torch.Tensor          # [P, m] float32
    needle_pos: list         # per unit: sorted absolute positions of planted keys


def generate(cfg: Config, device="cpu", seed: Optional[int] = None,
             unit_block: int = 64) -> Inputs:
    """Draw all inputs of `cfg` on `device` from one seeded generator.

    Draw order (fixed): W, b, queries, then per block of units: needle
    positions, offsets, keys, needle noise, values.  Keys and values are drawn
    in float32 and rounded to the storage dtype (round-to-nearest-even).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed if seed is None else seed)
    f32 = torch.float32
    U, G, d, m, P = cfg.U, cfg.G, cfg.d, cfg.m, cfg.P

    std = 1.0 / math.sqrt(d)      # W, b ~ N(0, 1/d)
    W = torch.randn(P, m, d, generator=g, device=dev, dtype=f32) * std
    b = torch.randn(P, m, generator=g, device=dev, dtype=f32) * std

    q = torch.randn(cfg.steps, U, G, d, generator=g, device=dev, dtype=f32)
    scales = torch.tensor([query_scale(cfg, u) for u in range(U)], device=dev, dtype=f32)
    q *= scales.view(1, U, 1, 1)

    kvdt = cfg.torch_kv_dtype()
    T = cfg.T_cap
    k = torch.empty(U, T, d, device=dev, dtype=kvdt)
    v = torch.empty(U, T, d, device=dev, dtype=kvdt)
    nn = n_needles(cfg)
    needle_pos = []
    q0 = q[0]
    qhat = q0 / q0.norm(dim=-1, keepdim=True)
    for u0 in range(0, U, unit_block):
        u1 = min(U, u0 + unit_block)
        nb = u1 - u0
        pos = []
        for u in range(u0, u1):
            perm = torch.randperm(cfg.L_mid, generator=g, device=dev)[:nn]
            pos.append(torch.sort(perm).values + cfg.n_sink)
        pos_t = torch.stack(pos) if nn > 0 else torch.zeros(nb, 0, dtype=torch.long, device=dev)
        if cfg.key_offset_norm > 0:
            xi = torch.randn(nb, d, generator=g, device=dev, dtype=f32)
            off = cfg.key_offset_norm * xi / xi.norm(dim=-1, keepdim=True)
        else:
            off = torch.zeros(nb, d, device=dev, dtype=f32)
        kb = torch.randn(nb, T, d, generator=g, device=dev, dtype=f32) + off[:, None, :]
        if cfg.needle_mode == "planted3":
            # three identical keys 4*q/|q| of query head 0 (exact ties)
            tgt = 4.0 * qhat[u0:u1, 0, :]
            for i in range(nb):
                kb[i, pos_t[i]] = tgt[i]
        elif nn > 0:
            j = torch.arange(nn, device=dev)
            gsel = j % G
            noise = 0.1 * torch.randn(nb, nn, d, generator=g, device=dev, dtype=f32)
            tgt = 4.0 * qhat[u0:u1][:, gsel, :] + noise       # [nb, nn, d]
            idx = pos_t[:, :, None].expand(nb, nn, d)
            kb.scatter_(1, idx, tgt)
        vb = torch.randn(nb, T, d, generator=g, device=dev, dtype=f32)
        k[u0:u1] = kb.to(kvdt)
        v[u0:u1] = vb.to(kvdt)
        needle_pos.extend([p.tolist() for p in pos_t.cpu()])
        del kb, vb
    return Inputs(cfg, k, v, q, W, b, needle_pos)


def unit_to_host(inp: Inputs, units: Sequence[int]):
    """Copy the per-unit slices of `inp` to host float32 tensors."""
    cfg = inp.cfg
    out = []
    for u in units:
        p = u % cfg.P
        out.append(dict(
            unit=u,
            k=inp.k[u].float().cpu(),
            v=inp.v[u].float().cpu(),
            q=inp.q[:, u].cpu(),
            W=inp.W[p].cpu(),
            b=inp.b[p].cpu(),
        ))
    return out


def generate_phi_mlp(cfg: Config, which: str, m: int = 64, device="cpu",
                     seed: Optional[int] = None) -> dict:
    """Random weights of the MLP feature maps (width 512, the pages' family; no
    training): one map per kv head for which="k" (cfg.P sets), one per query
    head for which="q" (cfg.P * cfg.G sets, query head (u, g) -> u % P * G + g).

    Scales keep every layer near unit variance: W_in ~ N(0, 1/d), W_1 ~
    N(0, 2/512), W_2 ~ N(0, 1/512), W_o ~ N(0, 0.25/512), biases ~ N(0, 0.01),
    alpha ~ U(0.25, 0.75), so the exponent W_o h1 + b_o stays within a few
    units and the features within about [0.05, 20].  Own generator (seed
    cfg.seed + 1000 for keys, + 2000 for queries): the other draws of the
    workload do not change.
    """
    n_sets = cfg.P if which == "k" else cfg.P * cfg.G
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((cfg.seed + (1000 if which == "k" else 2000)) if seed is None else seed)
    f32, H, d = torch.float32, 512, cfg.d

    def rn(*shape, std):
        return torch.randn(*shape, generator=g, device=dev, dtype=f32) * std
    return dict(W_in=rn(n_sets, H, d, std=1.0 / math.sqrt(d)), b_in=rn(n_sets, H, std=0.1),
                W_1=rn(n_sets, H, H, std=math.sqrt(2.0 / H)), b_1=rn(n_sets, H, std=0.1),
                W_2=rn(n_sets, H, H, std=1.0 / math.sqrt(H)), b_2=rn(n_sets, H, std=0.1),
                alpha=0.25 + 0.5 * torch.rand(n_sets, generator=g, device=dev, dtype=f32),
                W_o=rn(n_sets, m, H, std=0.5 / math.sqrt(H)), b_o=rn(n_sets, m, std=0.1))
