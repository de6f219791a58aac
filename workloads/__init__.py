"""Seeded synthetic inputs for grouped-query attention workloads.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and allocates tensors: it holds none of the attention
arithmetic, so neither the CPU oracle nor the HIP library depends on the other
through it.

Value distributions follow the problem statement: query, key and value entries
are standard normal, router logits are standard normal per (token, head), and
decode cache lengths are uniform integers in an inclusive range. Values are
drawn in float32 from a seeded ``torch.Generator`` and, for bfloat16 workloads,
rounded to bfloat16 (round-to-nearest-even, torch's cast).

Draw order for one workload is fixed: q, k, v, then lens (decode) or router
logits (routed prefill), so a seed names one input set exactly.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "prefill_inputs",
    "decode_inputs",
    "router_logits",
    "gqe_inputs",
    "torch_dtype",
    "GQE_SWEEP_T",
    "gqe_sweep_points",
    "router_inputs",
    "ROUTER_D_MODEL",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass(frozen=True)
class Workload:
    """One named synthetic workload (sizes, dtype and seed)."""

    name: str
    kind: str  # "prefill" | "decode" | "gqe"
    B: int
    h: int
    g: int
    T: int
    d: int
    dtype: str
    seed: int
    causal: bool = True
    lens: tuple[int, int] | None = None  # decode: inclusive range of cache lengths
    top_k: tuple[int, ...] = field(default_factory=tuple)  # gqe: the k values run
    g_sweep: tuple[int, ...] = field(default_factory=tuple)  # decode: KV-head counts run


# The five workloads of the problem statement. T is the sequence length for
# prefill and the cache capacity (T_max) for decode.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "prefill", B=1, h=4, g=2, T=16, d=16,
                         dtype="f32", seed=1, g_sweep=(2, 4, 1)),
    "prefill": Workload("prefill", "prefill", B=4, h=32, g=8, T=2048, d=128,
                        dtype="bf16", seed=2),
    "decode": Workload("decode", "decode", B=64, h=32, g=8, T=8192, d=128,
                       dtype="bf16", seed=3, lens=(1024, 8192)),
    "decode_sweep": Workload("decode_sweep", "decode", B=32, h=32, g=8, T=16384,
                             d=128, dtype="bf16", seed=4, lens=(16384, 16384),
                             g_sweep=(1, 4, 8, 32)),
    "gqe": Workload("gqe", "gqe", B=2, h=32, g=8, T=4096, d=128, dtype="bf16",
                    seed=5, top_k=(1, 2)),
}

# GQE-vs-GQA speed-up over the sequence length: the pages report the routed
# model's speed-up for 2k to 1024k-token sequences (gist.science GQE explainer,
# section "Resultats Experimentaux"). Every point holds GQE_SWEEP_TOKENS tokens
# (B = tokens / T, at least 1) so short sequences still fill the chip. Head
# shapes: the pages' 16 query heads over 8 KV groups with k = 1, and the
# 32-head / 8-group shape of the GQE workload with k = 1 and 2.
GQE_SWEEP_T = (2048, 4096, 8192, 16384, 32768, 65536)
GQE_SWEEP_TOKENS = 32768
GQE_SWEEP_SHAPES = ((16, 8, (1,)), (32, 8, (1, 2)))  # (h, g, top_k values)
GQE_SWEEP_D = 128
GQE_SWEEP_SEED = 6


def gqe_sweep_points():
    """(B, h, g, T, d, top_k values, seed) for every point of the sweep."""
    pts = []
    for h, g, ks in GQE_SWEEP_SHAPES:
        for T in GQE_SWEEP_T:
            B = max(1, GQE_SWEEP_TOKENS // T)
            pts.append((B, h, g, T, GQE_SWEEP_D, ks, GQE_SWEEP_SEED + T + h))
    return pts


# Router projection: the pages give neither the router's form nor the model
# width; the GQE workload's tokens (B=2, T=4096) are projected from
# d_model = h * d = 32 * 128 = 4096, the width whose projections give the
# query heads.
ROUTER_D_MODEL = 4096


def _gen(seed: int, device: str | torch.device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def _normal(shape, gen, device, dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def prefill_inputs(B: int, h: int, g: int, T: int, d: int, dtype: str = "bf16",
                   seed: int = 0, device: str | torch.device = "cpu"):
    """q [B,h,T,d], k [B,g,T,d], v [B,g,T,d], entries N(0,1) rounded to ``dtype``."""
    dt = torch_dtype(dtype)
    gen = _gen(seed, device)
    q = _normal((B, h, T, d), gen, device, dt)
    k = _normal((B, g, T, d), gen, device, dt)
    v = _normal((B, g, T, d), gen, device, dt)
    return q, k, v


def decode_inputs(B: int, h: int, g: int, T_max: int, d: int, lens_range,
                  dtype: str = "bf16", seed: int = 0,
                  device: str | torch.device = "cpu", poison_padding: bool = False):
    """One decode step over a KV cache.

    Returns q [B,h,d], k_cache [B,g,T_max,d], v_cache [B,g,T_max,d] and
    lens [B] (int32, uniform in the inclusive ``lens_range``). With
    ``poison_padding`` every cache slot at or beyond ``lens[b]`` holds NaN, so a
    kernel that reads past the valid length shows it in its output.
    """
    dt = torch_dtype(dtype)
    gen = _gen(seed, device)
    q = _normal((B, h, d), gen, device, dt)
    k = _normal((B, g, T_max, d), gen, device, dt)
    v = _normal((B, g, T_max, d), gen, device, dt)
    lo, hi = lens_range
    lens = torch.randint(lo, hi + 1, (B,), generator=gen, device=device,
                         dtype=torch.int64).to(torch.int32)
    if poison_padding:
        pos = torch.arange(T_max, device=device).view(1, 1, T_max, 1)
        pad = pos >= lens.view(B, 1, 1, 1).to(pos.dtype)
        k.masked_fill_(pad, float("nan"))
        v.masked_fill_(pad, float("nan"))
    return q, k, v, lens


def _logits(B, T, h, gen, device, ties):
    x = torch.randn(B, T, h, generator=gen, device=device, dtype=torch.float32)
    if ties:
        x = torch.round(x * 2.0) / 2.0
    return x


def router_logits(B: int, T: int, h: int, seed: int = 0,
                  device: str | torch.device = "cpu", ties: bool = False):
    """Router logits [B,T,h] float32, N(0,1).

    With ``ties`` the values are rounded to multiples of 1/2 so that equal
    logits inside one KV group are common (exercises the lower-index rule).
    """
    return _logits(B, T, h, _gen(seed, device), device, ties)


def gqe_inputs(B: int, h: int, g: int, T: int, d: int, dtype: str = "bf16",
               seed: int = 0, device: str | torch.device = "cpu",
               ties: bool = False):
    """q, k, v as in :func:`prefill_inputs`, then router logits [B,T,h] from
    the same generator."""
    dt = torch_dtype(dtype)
    gen = _gen(seed, device)
    q = _normal((B, h, T, d), gen, device, dt)
    k = _normal((B, g, T, d), gen, device, dt)
    v = _normal((B, g, T, d), gen, device, dt)
    return q, k, v, _logits(B, T, h, gen, device, ties)


def router_inputs(n_tok: int, d_model: int, h: int, seed: int = 0,
                  device: str | torch.device = "cpu"):
    """Router projection inputs: x [n_tok, d_model] ~ N(0,1) and router weights
    w_r [h, d_model] ~ N(0, 1/d_model), both rounded to bfloat16, so that the
    logits x w_r^T are about N(0,1) like the GQE workload's router logits."""
    gen = _gen(seed, device)
    x = _normal((n_tok, d_model), gen, device, torch.bfloat16)
    w = torch.randn(h, d_model, generator=gen, device=device, dtype=torch.float32)
    return x, (w / d_model ** 0.5).to(torch.bfloat16)
