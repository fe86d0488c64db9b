"""Seeded synthetic workloads for the MoE layer forward.

This module only describes shapes and draws random numbers; it holds none of
the layer's arithmetic.  Both the GPU path and the CPU oracle are fed from it.
The noisy router's standard-normal draws are not inputs: the library makes
them from the workload's rng_seed and rng_offset, and the oracle makes the
same ones from its own implementation of the same counter-based generator.

Distributions follow the workload descriptions: U ~ N(0, 1); router and
gate/up weights ~ N(0, 1/h); down weights ~ N(0, 1/f); the Switch-style
workload adds a per-expert logit bias ~ N(0, 1.5); the noisy workload adds a
noise-router weight ~ N(0, 1/h).  The second parameter of N(., .) is a
variance.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    h: int
    f: int
    E: int
    k: int
    dtype: str              # "f32" or "bf16"
    score: str              # "softmax" or "sigmoid"
    gate: str               # "raw" or "renorm"
    capacity_factor: float
    noisy: bool = False
    bias_var: float = 0.0   # variance of the per-expert logit bias (0: no bias)
    cap_mode: str = "assignments"
    fill: str = "rank_major"
    min_capacity: int = 0
    # DeepSeek-V3 parts (0: off): group-limited selection, shared experts and
    # the variance of the selection-only expert bias b_sel
    n_groups: int = 0
    topk_groups: int = 0
    n_shared: int = 0
    f_shared: int = 0
    sel_bias_var: float = 0.0
    # FP8 dispatch and up-projection (E4M3, power-of-two row scales); the
    # inputs stay bf16 and the weights are quantised once before the forward
    fp8_up: bool = False
    # noisy routing: key and counter offset of the standard-normal draws
    rng_seed: int = 0
    rng_offset: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny fp32 check, Mixtral shape, Switch-style top-1 with a
# skewing bias, DeepSeek-V3 fine-grained shape, and noisy top-2 at long batch.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=256, h=128, f=256, E=8, k=2, dtype="f32",
                         score="softmax", gate="renorm", capacity_factor=1.25),
    "mixtral_bf16": Workload("mixtral_bf16", T=4096, h=4096, f=14336, E=8, k=2,
                             dtype="bf16", score="softmax", gate="renorm",
                             capacity_factor=1.25),
    "switch_bf16": Workload("switch_bf16", T=8192, h=1024, f=4096, E=128, k=1,
                            dtype="bf16", score="softmax", gate="raw",
                            capacity_factor=1.25, bias_var=1.5),
    "deepseek_v3_bf16": Workload("deepseek_v3_bf16", T=4096, h=7168, f=2048, E=256, k=8,
                                 dtype="bf16", score="sigmoid", gate="renorm",
                                 capacity_factor=2.0),
    "noisy_long_bf16": Workload("noisy_long_bf16", T=32768, h=4096, f=14336, E=64, k=2,
                                dtype="bf16", score="softmax", gate="renorm",
                                capacity_factor=1.0, noisy=True),
    # the DeepSeek-V3 shape with its layer parts: 1 shared expert of the same
    # width, node-limited selection (8 groups, at most 4 per token) and a
    # selection bias with standard deviation 0.01
    "deepseek_v3_full_bf16": Workload("deepseek_v3_full_bf16", T=4096, h=7168, f=2048, E=256,
                                      k=8, dtype="bf16", score="sigmoid", gate="renorm",
                                      capacity_factor=2.0, n_groups=8, topk_groups=4,
                                      n_shared=1, f_shared=2048, sel_bias_var=1e-4),
    # the Mixtral shape with the FP8 dispatch and up-projection
    "mixtral_fp8": Workload("mixtral_fp8", T=4096, h=4096, f=14336, E=8, k=2, dtype="bf16",
                            score="softmax", gate="renorm", capacity_factor=1.25, fp8_up=True),
}

WORKLOAD_ORDER = ["tiny_f32", "mixtral_bf16", "switch_bf16", "deepseek_v3_bf16",
                  "noisy_long_bf16"]


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _normal(shape, var, gen, device, out_dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if var != 1.0:
        x.mul_(math.sqrt(var))
    return x.to(out_dtype)


def make_inputs(w: Workload, seed: int = 0, device="cpu", with_experts: bool = True) -> dict:
    """Draw every input of workload w from one seeded generator, in a fixed order.

    Expert weights are drawn one expert at a time so that large workloads never
    hold a float32 copy of all weights.  Shapes: U [T, h]; W_r, W_noise [h, E];
    b_r [E] fp32; b_sel [E] fp32; W_gate, W_up [E, f, h];
    W_down [E, h, f]; Ws_gate, Ws_up [n_shared, f_shared, h]; Ws_down
    [n_shared, h, f_shared].  Inputs a workload does not use are None and draw
    nothing, so adding a part never changes the other inputs.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = torch_dtype(w)
    x = {}
    x["U"] = _normal((w.T, w.h), 1.0, gen, dev, dt)
    x["W_r"] = _normal((w.h, w.E), 1.0 / w.h, gen, dev, dt)
    x["b_r"] = _normal((w.E,), w.bias_var, gen, dev, torch.float32) if w.bias_var > 0 else None
    x["W_noise"] = _normal((w.h, w.E), 1.0 / w.h, gen, dev, dt) if w.noisy else None
    x["b_sel"] = (_normal((w.E,), w.sel_bias_var, gen, dev, torch.float32)
                  if w.sel_bias_var > 0 else None)
    if with_experts:
        x["W_gate"] = torch.empty((w.E, w.f, w.h), dtype=dt, device=dev)
        x["W_up"] = torch.empty((w.E, w.f, w.h), dtype=dt, device=dev)
        x["W_down"] = torch.empty((w.E, w.h, w.f), dtype=dt, device=dev)
        for e in range(w.E):
            x["W_gate"][e] = _normal((w.f, w.h), 1.0 / w.h, gen, dev, dt)
            x["W_up"][e] = _normal((w.f, w.h), 1.0 / w.h, gen, dev, dt)
            x["W_down"][e] = _normal((w.h, w.f), 1.0 / w.f, gen, dev, dt)
    x["Ws_gate"] = x["Ws_up"] = x["Ws_down"] = None
    if with_experts and w.n_shared > 0:
        fs = w.f_shared
        x["Ws_gate"] = torch.empty((w.n_shared, fs, w.h), dtype=dt, device=dev)
        x["Ws_up"] = torch.empty((w.n_shared, fs, w.h), dtype=dt, device=dev)
        x["Ws_down"] = torch.empty((w.n_shared, w.h, fs), dtype=dt, device=dev)
        for i in range(w.n_shared):
            x["Ws_gate"][i] = _normal((fs, w.h), 1.0 / w.h, gen, dev, dt)
            x["Ws_up"][i] = _normal((fs, w.h), 1.0 / w.h, gen, dev, dt)
            x["Ws_down"][i] = _normal((w.h, fs), 1.0 / fs, gen, dev, dt)
    return x
