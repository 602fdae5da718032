"""Seeded synthetic inputs for the routed fused-MoE expert FFN.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the method's arithmetic: it only draws a routing (expert ids
per token), routed weights, token rows and expert weights.  Building the
dispatch contract, packing and the FFN itself are done separately by the
oracle and by the HIP library.

Recipe:
  * routing: every token picks k distinct experts.  The tiny case uses
    CPython ``random.Random(seed).sample(range(E), k)`` per token, as the
    tutorial's contract script does.  The others draw per-token successive
    sampling without replacement with expert probabilities p (uniform, or
    Zipf p_e ~ (e+1)^-s with expert 0 the most popular) through the
    Gumbel-top-k construction on ``numpy.random.default_rng(seed)``.
  * routed weights: fp32 softmax over the k slots of N(0,1) logits.
  * tokens x ~ N(0,1) -> fp16; Wg, Wu ~ N(0, 1/H) -> fp16 with layout
    [E, I, H]; Wd ~ N(0, 1/I) -> fp16 with layout [E, H, I].
  * tensors come from ``torch.Generator`` streams seeded per tensor, on the
    device asked for (CPU for the small cases, the GPU for the big ones so
    that 11 GB of weights appear in milliseconds).
"""
from __future__ import annotations

import dataclasses
import math
import random

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    tokens: int
    experts: int
    top_k: int
    hidden: int
    intermediate: int
    routing: str = "uniform"      # "uniform", "zipf", "pysample"
    zipf_s: float = 0.0
    seed: int = 7

    @property
    def pairs(self) -> int:
        return self.tokens * self.top_k

    @property
    def num_blocks_m(self) -> int:
        return -(-self.pairs // 128) + self.experts

    def useful_flops(self) -> float:
        """6 * pairs * H * I: two GEMMs of 2*H*I per pair for gate/up and one
        for down."""
        return 6.0 * self.pairs * self.hidden * self.intermediate


CONFIGS = {
    "tiny": Config("tiny", 9, 4, 2, 256, 128, routing="pysample"),
    "decode": Config("decode", 64, 8, 2, 4096, 14336),
    "prefill": Config("prefill", 4096, 8, 2, 4096, 14336),
    "fine": Config("fine", 8192, 64, 6, 2048, 1408, routing="zipf", zipf_s=1.1),
    "large": Config("large", 16384, 128, 8, 7168, 2048, routing="zipf", zipf_s=1.2),
}


def draw_routing(cfg: Config) -> np.ndarray:
    """topk_ids [T, k] int32, k distinct experts per token."""
    T, E, k = cfg.tokens, cfg.experts, cfg.top_k
    if k > E:
        raise ValueError("top_k exceeds the number of experts")
    if cfg.routing == "pysample":
        rng = random.Random(cfg.seed)
        return np.array([rng.sample(range(E), k) for _ in range(T)], dtype=np.int32).reshape(T, k)
    rng = np.random.default_rng(cfg.seed)
    if cfg.routing == "uniform":
        logp = np.zeros(E)
    elif cfg.routing == "zipf":
        w = (np.arange(E) + 1.0) ** (-cfg.zipf_s)
        logp = np.log(w / w.sum())
    else:
        raise ValueError(cfg.routing)
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return np.ascontiguousarray(ids, dtype=np.int32)


def routing_from_counts(counts, seed: int = 7) -> np.ndarray:
    """k=1 routing where expert e receives exactly counts[e] tokens, in a
    seeded random token order.  For edge cases (empty experts, groups of
    127/128/129/256 rows)."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(seed).shuffle(ids)
    return ids.reshape(-1, 1).astype(np.int32)


def draw_routed_weights(T: int, k: int, seed: int) -> np.ndarray:
    """fp32 softmax over the k slots of N(0,1) logits, per token."""
    rng = np.random.default_rng([seed, 1])
    logits = rng.standard_normal((T, k)).astype(np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)


def _gen(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + tag)
    return g


def _normal_f16(shape, std, seed, tag, device, chunks=1) -> torch.Tensor:
    """fp16 tensor of N(0, std^2) values, drawn in fp32 chunk by chunk along
    dim 0 (to bound the fp32 temporary) and rounded to nearest fp16."""
    out = torch.empty(shape, dtype=torch.float16, device=device)
    g = _gen(seed, tag, device)
    n0 = shape[0]
    step = max(1, -(-n0 // chunks))
    for a in range(0, n0, step):
        b = min(n0, a + step)
        tmp = torch.randn((b - a,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        out[a:b] = (tmp * std).to(torch.float16)
    return out


@dataclasses.dataclass
class Inputs:
    cfg: Config
    topk_ids: np.ndarray          # [T, k] int32
    topk_w: np.ndarray            # [T, k] float32
    x: torch.Tensor               # [T, H] fp16
    wg: torch.Tensor              # [E, I, H] fp16
    wu: torch.Tensor              # [E, I, H] fp16
    wd: torch.Tensor              # [E, H, I] fp16


def make_inputs(cfg: Config, device="cpu", topk_ids: np.ndarray | None = None) -> Inputs:
    """All inputs of one workload.  ``topk_ids`` overrides the routing (the
    token count then follows it)."""
    if topk_ids is None:
        topk_ids = draw_routing(cfg)
    T, k = topk_ids.shape
    E, H, I = cfg.experts, cfg.hidden, cfg.intermediate
    topk_w = draw_routed_weights(T, k, cfg.seed)
    big = E * I * H > (1 << 26)
    ch = E if big else 1
    x = _normal_f16((T, H), 1.0, cfg.seed, 1, device, chunks=max(1, T // 4096))
    wg = _normal_f16((E, I, H), 1.0 / math.sqrt(H), cfg.seed, 2, device, chunks=ch)
    wu = _normal_f16((E, I, H), 1.0 / math.sqrt(H), cfg.seed, 3, device, chunks=ch)
    wd = _normal_f16((E, H, I), 1.0 / math.sqrt(I), cfg.seed, 4, device, chunks=ch)
    return Inputs(cfg, topk_ids, topk_w, x, wg, wu, wd)


def make_router_weight(cfg: Config, device="cpu") -> torch.Tensor:
    """Synthetic router gate [E, H] fp16, N(0, 1/H): with x ~ N(0, 1) the
    logits are ~N(0, 1), a spread of scores like a trained router's."""
    return _normal_f16((cfg.experts, cfg.hidden), 1.0 / math.sqrt(cfg.hidden), cfg.seed, 5, device)

