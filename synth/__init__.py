"""Seeded synthetic inputs for the MoE decode layer.

This module is shared by the tests, the benchmark and the smoke check. It
holds the workload table and the random draws only: none of the layer's
arithmetic (no projection, routing, activation or normalisation) lives here,
so the oracle and the HIP path stay independent of each other and of it.

Every tensor comes from its own generator stream, seeded by
``stream_seed(seed, name, index)``, so any single expert's weights can be
drawn again without drawing the rest. Floating-point draws are made in fp32
and rounded to bf16 with torch's round-to-nearest-even conversion.

Workloads (shapes and value distributions) follow the decode shapes of the
"Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly" post
(Part 1, sections 1-4: batch 1-64 decode, router + latent projection, routed
and shared experts, attention input/output projections with residual); the
pages give no model dimensions, so the sizes below are the workload table of
this library (d = 7168, E = 384, top-8, I = 2048).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "MoEConfig", "ChainConfig", "MOE_CONFIGS", "CHAIN_CONFIG", "CHAIN_BATCHES",
    "stream_seed", "randn_bf16", "uniform_bf16", "zipf_router_bias",
    "make_moe_weights", "make_tokens", "make_chain_weights", "make_chain_inputs",
]


@dataclass(frozen=True)
class MoEConfig:
    """One MoE block workload: b tokens of width d routed top-k over E experts."""
    name: str
    b: int
    d: int
    E: int
    k: int
    I: int          # routed expert SwiGLU intermediate size
    I_s: int        # shared expert SwiGLU intermediate size
    d_lat: int      # latent projection output width (= expert input width)
    zipf_bias: float = 0.0   # Zipf exponent of the router bias; 0 = no bias
    seed: int = 0

    @property
    def w_std(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def router_bound(self) -> float:
        # uniform router weights with variance 1/d: U(-sqrt(3/d), sqrt(3/d))
        return math.sqrt(3.0 / self.d)


@dataclass(frozen=True)
class ChainConfig:
    """Attention input projection K_in -> N_in, then output projection
    K_o -> d with residual add and RMSNorm."""
    name: str
    d: int = 7168
    n_in: int = 12288
    k_o: int = 8192
    eps: float = 1e-6
    seed: int = 0


MOE_CONFIGS = {
    "tiny": MoEConfig("tiny", b=1, d=256, E=8, k=2, I=128, I_s=128, d_lat=256),
    "b1": MoEConfig("b1", b=1, d=7168, E=384, k=8, I=2048, I_s=2048, d_lat=7168),
    "b16": MoEConfig("b16", b=16, d=7168, E=384, k=8, I=2048, I_s=2048, d_lat=7168),
    "b64zipf": MoEConfig("b64zipf", b=64, d=7168, E=384, k=8, I=2048, I_s=2048, d_lat=7168,
                         zipf_bias=1.1),
    # one GPU's share of the experts under tensor parallelism over 8 GPUs
    # (I = I_s = 2048 / 8); router and latent rows whole
    "tp8_shard": MoEConfig("tp8_shard", b=1, d=7168, E=384, k=8, I=256, I_s=256, d_lat=7168),
}
CHAIN_CONFIG = ChainConfig("chain")
CHAIN_BATCHES = (1, 2, 4, 8, 16, 32, 64)


def stream_seed(seed: int, name: str, index: int = 0) -> int:
    """63-bit seed of the generator stream for tensor `name` (part `index`)."""
    h = hashlib.sha256(f"k3dec/{seed}/{name}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, name, index):
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, name, index))
    return g


def randn_bf16(shape, std, seed, name, index=0, device="cpu", out=None):
    """N(0, std^2) draws, fp32 then rounded to bf16 (RNE). Writes into `out` if given."""
    g = _gen(device, seed, name, index)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    if out is not None:
        out.copy_(t)
        return out
    return t.to(torch.bfloat16)


def uniform_bf16(shape, bound, seed, name, index=0, device="cpu"):
    """U(-bound, bound) draws, fp32 then rounded to bf16 (RNE)."""
    g = _gen(device, seed, name, index)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(2.0 * bound).sub_(bound)
    return t.to(torch.bfloat16)


def zipf_router_bias(E: int, s: float, seed: int) -> torch.Tensor:
    """fp32 router bias b_e = -s * ln(rank_e), rank = 1 + a seeded permutation.

    exp(b_e) = rank_e^(-s): a Zipf(s) popularity over the experts, applied as
    an additive logit bias, so a few experts draw many tokens.
    """
    g = _gen("cpu", seed, "router_bias_perm", 0)
    rank = torch.randperm(E, generator=g).to(torch.float64) + 1.0
    return (-s * torch.log(rank)).to(torch.float32)


def make_moe_weights(cfg: MoEConfig, device="cpu", layer: int = 0) -> dict:
    """All weights of one MoE block, [out x in] row-major, bf16 (bias fp32).

    w13[e] stacks the gate rows [0, I) over the up rows [I, 2I).
    `layer` selects an independent draw (distinct layers of a model stack).
    """
    s = cfg.seed + 1000003 * layer
    d, E, I, Is, dl = cfg.d, cfg.E, cfg.I, cfg.I_s, cfg.d_lat
    w = {}
    w["w_router"] = uniform_bf16((E, d), cfg.router_bound, s, "w_router", device=device)
    w["bias"] = (zipf_router_bias(E, cfg.zipf_bias, s).to(device)
                 if cfg.zipf_bias > 0 else None)
    w["w_lat"] = randn_bf16((dl, d), cfg.w_std, s, "w_lat", device=device)
    w13 = torch.empty((E, 2 * I, dl), dtype=torch.bfloat16, device=device)
    w2 = torch.empty((E, d, I), dtype=torch.bfloat16, device=device)
    for e in range(E):
        randn_bf16((2 * I, dl), cfg.w_std, s, "w13", e, device=device, out=w13[e])
        randn_bf16((d, I), cfg.w_std, s, "w2", e, device=device, out=w2[e])
    w["w13"] = w13
    w["w2"] = w2
    w["w13_s"] = randn_bf16((2 * Is, d), cfg.w_std, s, "w13_s", device=device)
    w["w2_s"] = randn_bf16((d, Is), cfg.w_std, s, "w2_s", device=device)
    return w


def make_tokens(cfg: MoEConfig, device="cpu", index: int = 0, b: int | None = None):
    """x ~ N(0, 1), [b x d] bf16. `index` selects an independent batch."""
    b = cfg.b if b is None else b
    return randn_bf16((b, cfg.d), 1.0, cfg.seed, "x", index, device=device)


def make_chain_weights(cfg: ChainConfig = CHAIN_CONFIG, device="cpu", layer: int = 0) -> dict:
    """W_in [n_in x d], W_o [d x k_o] ~ N(0, 1/K); gamma = 1 + 0.1 N(0,1), bf16."""
    s = cfg.seed + 1000003 * layer
    w = {}
    w["w_in"] = randn_bf16((cfg.n_in, cfg.d), 1.0 / math.sqrt(cfg.d), s, "w_in", device=device)
    w["w_o"] = randn_bf16((cfg.d, cfg.k_o), 1.0 / math.sqrt(cfg.k_o), s, "w_o", device=device)
    g = randn_bf16((cfg.d,), 0.1, s, "gamma", device=device).float() + 1.0
    w["gamma"] = g.to(torch.bfloat16)
    return w


def make_chain_inputs(cfg: ChainConfig, b: int, device="cpu", index: int = 0) -> dict:
    """x, r ~ N(0, 1), [b x d] bf16."""
    return {
        "x": randn_bf16((b, cfg.d), 1.0, cfg.seed, "chain_x", index, device=device),
        "r": randn_bf16((b, cfg.d), 1.0, cfg.seed, "chain_r", index, device=device),
    }
