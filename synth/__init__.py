"""Seeded synthetic inputs for the BFP4/BFP8 weight-streaming matmul workloads.

This module only draws random numbers. It holds none of the block-floating-point
arithmetic (no exponent sharing, no mantissa rounding, no matmul): both the CPU
oracle's tests and the GPU path's tests and bench take their inputs from here.

The pages' workloads are whole Qwen-family models on text corpora; none of that is
needed or reproduced here. These generators stand in for trained weights with the
shapes and value distributions of the five workloads studied:

* single BFP8 GEMV 2048x2048 (weights N(0, 0.02) x per-output-column LogNormal(0, 0.5),
  0.1% outliers x20),
* dense BFP4 MLP at 27B-class shapes (5120 -> 17408 gate/up, 17408 -> 5120 down),
* BFP8 fused QKV projection, output projection and LM head at decode,
* a 256-expert top-8 MoE layer with a shared expert (decode and a 2048-token prefill
  chunk with a skewed per-expert router bias).

Every tensor is drawn from its own stream, ``default_rng(SeedSequence([seed, cfg_id,
crc32(name)]))``, so draws do not depend on the order in which tensors are made.
Matrices are drawn directly in their stored orientation ``[N][K]`` (output rows,
reduction along K); the per-output-column scale of the K x N formulation is therefore a
per-row scale here. Activations are drawn in fp32 and rounded to bf16 (round to
nearest, ties to even) and returned as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = [
    "rng_for", "bf16_bits", "bf16_values", "normal_bf16", "dense_weights",
    "gemv_case", "mlp_case", "proj_case", "moe_router", "moe_layer", "moe_tokens", "router_bias",
    "HIDDEN", "INTER", "N_EXPERTS", "TOP_K",
]

# MoE layer shape of the 35B-A3B family: 256 routed experts, top-8, one shared expert.
HIDDEN = 2048
INTER = 512
N_EXPERTS = 256
TOP_K = 8


def rng_for(seed: int, cfg_id: int, name: str) -> np.random.Generator:
    """Independent generator for one named tensor of one workload."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(cfg_id), zlib.crc32(name.encode())]))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_values(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def dense_weights(seed: int, cfg_id: int, name: str, n: int, k: int, std: float = 0.02,
                  row_sigma: float | None = None, outlier_p: float = 0.0,
                  outlier_mult: float = 20.0) -> np.ndarray:
    """fp32 [n][k]: N(0, std) x per-row LogNormal(0, row_sigma), optional Bernoulli outliers."""
    rng = rng_for(seed, cfg_id, name)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    if row_sigma is not None:
        s = rng.lognormal(0.0, row_sigma, size=(n, 1)).astype(np.float32)
        w *= s
    if outlier_p > 0.0:
        mask = rng.random((n, k), dtype=np.float32) < outlier_p
        w[mask] *= np.float32(outlier_mult)
    return w


def gemv_case(seed: int = 0, n: int = 2048, k: int = 2048, m: int = 1) -> dict:
    """Single BFP8 GEMV: x m x k bf16 N(0,1); W [n][k] with row scales and 0.1% x20 outliers."""
    w = dense_weights(seed, 1, "w", n, k, 0.02, row_sigma=0.5, outlier_p=0.001)
    x = normal_bf16(rng_for(seed, 1, "x"), (m, k))
    return {"fmt": 8, "x": x, "w": w}


def mlp_case(m: int, seed: int = 0, hidden: int = 5120, inter: int = 17408) -> dict:
    """Dense BFP4 MLP decode (27B-class): gate/up [inter][hidden], down [hidden][inter]."""
    return {
        "fmt": 4,
        "x": normal_bf16(rng_for(seed, 2, f"x{m}"), (m, hidden)),
        "wg": dense_weights(seed, 2, "gate", inter, hidden, 0.02, row_sigma=0.5),
        "wu": dense_weights(seed, 2, "up", inter, hidden, 0.02, row_sigma=0.5),
        "wd": dense_weights(seed, 2, "down", hidden, inter, 0.02, row_sigma=0.5),
    }


def proj_case(m: int, seed: int = 0, hidden: int = 2048, q_out: int = 4096, kv_out: int = 512,
              vocab: int = 151936, with_lm: bool = True) -> dict:
    """BFP8 fused QKV [q+2kv][hidden], output projection [hidden][q], LM head [vocab][hidden]."""
    d = {
        "fmt": 8,
        "x": normal_bf16(rng_for(seed, 3, f"x{m}"), (m, hidden)),
        "xo": normal_bf16(rng_for(seed, 3, f"xo{m}"), (m, q_out)),
        "wqkv": dense_weights(seed, 3, "qkv", q_out + 2 * kv_out, hidden, 0.02),
        "wo": dense_weights(seed, 3, "o", hidden, q_out, 0.02),
    }
    if with_lm:
        d["wlm"] = dense_weights(seed, 3, "lm", vocab, hidden, 0.02)
    return d


def moe_router(seed: int = 0, n_experts: int = N_EXPERTS, hidden: int = HIDDEN):
    """Router bf16 [E][hidden] N(0, 0.02) and shared-expert gate vector bf16 [hidden]."""
    router = normal_bf16(rng_for(seed, 4, "router"), (n_experts, hidden), std=0.02)
    sh_gate_w = normal_bf16(rng_for(seed, 4, "shared_gate"), (hidden,), std=0.02)
    return router, sh_gate_w


def moe_layer(seed: int = 0, n_experts: int = N_EXPERTS, hidden: int = HIDDEN, inter: int = INTER,
              experts: np.ndarray | None = None) -> dict:
    """One MoE layer: bf16 router [E][hidden], stacked expert weights, shared expert.

    Expert weights are N(0, 0.02) x a_e with a_e ~ LogNormal(0, 0.3) per expert (one
    scalar for that expert's gate, up and down). Stacking is along the output rows:
    gate/up are [E*inter][hidden] and down is [E*hidden][inter]. If ``experts`` is
    given, only those experts' weights are drawn (the others stay zero): this lets tiny
    CPU tests build the few experts they route to without drawing all 256.
    """
    cfg = 4  # the decode and prefill workloads share one layer
    router, sh_gate_w = moe_router(seed, n_experts, hidden)
    scales = rng_for(seed, cfg, "expert_scale").lognormal(0.0, 0.3, size=n_experts + 1).astype(np.float32)
    sel = np.arange(n_experts) if experts is None else np.unique(np.asarray(experts, dtype=np.int64))
    gate = np.zeros((n_experts * inter, hidden), np.float32)
    up = np.zeros((n_experts * inter, hidden), np.float32)
    down = np.zeros((n_experts * hidden, inter), np.float32)
    for e in sel:
        a = scales[e]
        gate[e * inter:(e + 1) * inter] = dense_weights(seed, cfg, f"gate{e}", inter, hidden) * a
        up[e * inter:(e + 1) * inter] = dense_weights(seed, cfg, f"up{e}", inter, hidden) * a
        down[e * hidden:(e + 1) * hidden] = dense_weights(seed, cfg, f"down{e}", hidden, inter) * a
    a = scales[n_experts]
    return {
        "fmt": 4, "n_experts": n_experts, "top_k": TOP_K, "hidden": hidden, "inter": inter,
        "router": router, "sh_gate_w": sh_gate_w,
        "gate": gate, "up": up, "down": down,
        "sh_gate": dense_weights(seed, cfg, "sh_gate", inter, hidden) * a,
        "sh_up": dense_weights(seed, cfg, "sh_up", inter, hidden) * a,
        "sh_down": dense_weights(seed, cfg, "sh_down", hidden, inter) * a,
        "drawn": sel,
    }


def moe_tokens(m: int, seed: int = 0, hidden: int = HIDDEN, cfg_id: int = 4) -> np.ndarray:
    """MoE input rows: m x hidden bf16 N(0, 1)."""
    return normal_bf16(rng_for(seed, cfg_id, f"x{m}"), (m, hidden))


def router_bias(seed: int = 0, n_experts: int = N_EXPERTS, std: float = 1.5) -> np.ndarray:
    """Skewed per-expert router-logit bias of the prefill workload, fp32 N(0, 1.5)."""
    return (rng_for(seed, 5, "bias").standard_normal(n_experts) * std).astype(np.float32)
