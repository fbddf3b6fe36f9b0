"""Seeded synthetic inputs for the MoE decode layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the GPU tests/benchmark and the CPU oracle's tests
take their inputs from here.

Recipe (the pages measure on real prompts and private/benchmark workloads that
are not available; these seeded draws stand in for them):

* weights: N(0, std) drawn in float32, rounded to bf16 by torch's conversion
  (round to nearest even); router std 0.02 unless the workload says otherwise;
* activations x: N(0, 1), one independent sub-stream per token and redraw
  number, so a single token can be redrawn without touching the others;
* router bias (skewed workload only): b_e = ln p_r(e), p_r proportional to
  r^-s over ranks r = 1..E (Zipf exponent s), ranks given to experts by a
  seeded permutation;
* host draws use NumPy PCG64 seeded by SeedSequence([seed, tensor_id, ...]);
  device draws use torch's CUDA generator seeded by seed*1000 + tensor_id, one
  expert at a time.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

SOFTMAX = 0
SIGMOID = 1

# tensor ids for sub-streams
T_X, T_WR, T_W13, T_W2, T_S13, T_S2, T_BIAS, T_SPEC_BASE, T_SPEC_OWN = range(9)

# Speculative-decoding verify batches: each request scores its draft tokens
# plus one (7 drafts in the Kimi K3 article's DSpark runs, Part 3), and the
# tokens of one request share a common direction with weight SPEC_RHO.
SPEC_TOKENS_PER_REQUEST = 8
SPEC_RHO = 0.5


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    batch: int
    score_fn: int
    router_std: float = 0.02
    weight_std: float = 0.02
    zipf_s: float | None = None
    seed: int = 0

    def with_batch(self, b: int) -> "Workload":
        return replace(self, batch=b)


# The five workloads the layer is specified on.
TINY = Workload("tiny_h256_e8_k2", 256, 8, 2, 128, 128, 1, SOFTMAX)
TP8 = Workload("tp8shard_h7168_e384_k8_i256", 7168, 384, 8, 256, 256, 1, SIGMOID)
TP8_UNIT = replace(TP8, name="tp8shard_unitlogit", router_std=1.0 / math.sqrt(7168))
TP8_ZIPF = replace(TP8, name="tp8shard_zipf1.1", batch=64, zipf_s=1.1)
FULL = Workload("unsharded_h7168_e384_k8_i2048", 7168, 384, 8, 2048, 2048, 32, SIGMOID)

WORKLOADS = {w.name: w for w in (TINY, TP8, TP8_UNIT, TP8_ZIPF, FULL)}


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded by torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def host_normal(shape, std: float, seed: int, *ids: int) -> np.ndarray:
    return f32_to_bf16_bits(_rng(seed, *ids).standard_normal(shape, dtype=np.float32) * np.float32(std))


def token_x(wl: Workload, t: int, redraw: int = 0) -> np.ndarray:
    """Activation row for token t (redraw number ``redraw``), bf16 bits [H]."""
    return host_normal((wl.hidden,), 1.0, wl.seed, T_X, t, redraw)


def spec_token_x(wl: Workload, t: int, redraw: int = 0, per_request: int = SPEC_TOKENS_PER_REQUEST,
                 rho: float = SPEC_RHO) -> np.ndarray:
    """Token t of a verify batch (requests of ``per_request`` consecutive
    tokens): sqrt(rho) * request base + sqrt(1 - rho) * the token's own draw,
    both ~N(0, 1), so each row keeps unit variance and rows of one request
    have correlation rho.  bf16 bits [H]; ``redraw`` redraws the own part."""
    H = wl.hidden
    base = _rng(wl.seed, T_SPEC_BASE, t // per_request).standard_normal(H, dtype=np.float32)
    own = _rng(wl.seed, T_SPEC_OWN, t, redraw).standard_normal(H, dtype=np.float32)
    return f32_to_bf16_bits(np.float32(math.sqrt(rho)) * base + np.float32(math.sqrt(1.0 - rho)) * own)


def spec_batch_x(wl: Workload, batch: int, offset: int = 0) -> np.ndarray:
    return np.stack([spec_token_x(wl, offset + t) for t in range(batch)])


def batch_x(wl: Workload, batch: int | None = None, offset: int = 0) -> np.ndarray:
    b = wl.batch if batch is None else batch
    return np.stack([token_x(wl, offset + t) for t in range(b)])


def zipf_bias(wl: Workload) -> np.ndarray | None:
    if wl.zipf_s is None:
        return None
    E = wl.n_experts
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-wl.zipf_s)
    p /= p.sum()
    perm = _rng(wl.seed, T_BIAS).permutation(E)      # expert perm[r] gets rank r+1
    b = np.empty(E, np.float32)
    b[perm] = np.log(p).astype(np.float32)
    return b


def host_layer(wl: Workload) -> dict:
    """All weights on the host as bf16 bits (tiny and medium shapes only)."""
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    d = {
        "wr": host_normal((E, H), wl.router_std, wl.seed, T_WR),
        "w13": np.stack([host_normal((2 * I, H), wl.weight_std, wl.seed, T_W13, e) for e in range(E)]),
        "w2": np.stack([host_normal((H, I), wl.weight_std, wl.seed, T_W2, e) for e in range(E)]),
        "bias": zipf_bias(wl),
    }
    if Is > 0:
        d["s13"] = host_normal((2 * Is, H), wl.weight_std, wl.seed, T_S13)
        d["s2"] = host_normal((H, Is), wl.weight_std, wl.seed, T_S2)
    else:
        d["s13"] = d["s2"] = None
    return d


def _dev_normal(n: int, std: float, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(std).to(torch.bfloat16)


def _dev_base(wl: Workload, layer: int) -> int:
    return (wl.seed * 1000 + layer * 16) * 1000


def device_router(wl: Workload, device="cuda", layer: int = 0) -> torch.Tensor:
    """The router weight [E x H] of ``device_layer(wl, device, layer)`` alone
    (bf16, N(0, wl.router_std)); workloads that differ only in router_std draw
    the same normal variates, scaled differently."""
    g = torch.Generator(device=device)
    g.manual_seed(_dev_base(wl, layer) + T_WR)
    return _dev_normal(wl.n_experts * wl.hidden, wl.router_std, g, device).view(wl.n_experts, wl.hidden)


def device_layer(wl: Workload, device="cuda", layer: int = 0) -> dict:
    """Weights drawn on the device in the GPU library's packed layout.

    expert_w = [W13: E x 2I x H][W2: E x H x I], shared_w = [S13: 2Is x H][S2: H x Is],
    router_w = [E x H]; all bf16.  ``layer`` selects an independent draw.
    """
    E, H, I, Is = wl.n_experts, wl.hidden, wl.inter, wl.shared_inter
    base = _dev_base(wl, layer)
    g = torch.Generator(device=device)
    wr = device_router(wl, device, layer)
    expert_w = torch.empty(E * 3 * I * H, dtype=torch.bfloat16, device=device)
    n13 = 2 * I * H
    for e in range(E):
        g.manual_seed(base + T_W13 * 100000 + e)
        expert_w[e * n13:(e + 1) * n13] = _dev_normal(n13, wl.weight_std, g, device)
    off2 = E * n13
    n2 = H * I
    for e in range(E):
        g.manual_seed(base + T_W2 * 100000 + e)
        expert_w[off2 + e * n2: off2 + (e + 1) * n2] = _dev_normal(n2, wl.weight_std, g, device)
    if Is > 0:
        g.manual_seed(base + T_S13)
        shared_w = torch.empty(3 * Is * H, dtype=torch.bfloat16, device=device)
        shared_w[:2 * Is * H] = _dev_normal(2 * Is * H, wl.weight_std, g, device)
        g.manual_seed(base + T_S2)
        shared_w[2 * Is * H:] = _dev_normal(Is * H, wl.weight_std, g, device)
    else:
        shared_w = torch.empty(0, dtype=torch.bfloat16, device=device)
    b = zipf_bias(wl)
    bias = None if b is None else torch.from_numpy(b).to(device)
    return {"router_w": wr, "expert_w": expert_w, "shared_w": shared_w, "bias": bias}


def pack_host_layer(d: dict) -> dict:
    """Host layer dict -> flat bf16-bit arrays in the GPU library's packed layout."""
    ew = np.concatenate([d["w13"].reshape(-1), d["w2"].reshape(-1)])
    sw = (np.concatenate([d["s13"].reshape(-1), d["s2"].reshape(-1)])
          if d["s13"] is not None else np.zeros(0, np.uint16))
    return {"router_w": d["wr"], "expert_w": ew, "shared_w": sw, "bias": d["bias"]}


def bits_to_torch_bf16(a: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def torch_bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
