"""Seeded synthetic workloads for the MoE FFN layer: shapes and input tensors.

This module only draws random numbers and lays out tensors. It holds no step
of the layer's arithmetic, so both the HIP path and the fp64 oracle can take
their inputs from it without sharing any of the method.

Recipe (the same for every workload):
  * every tensor (and every expert's slice of a per-expert tensor) has its own
    torch generator, seeded from (seed, tensor id, global expert index) through
    a splitmix64 mix, so any piece can be regenerated alone;
  * values are drawn as float32 standard normals times a standard deviation,
    then rounded to the I/O dtype (round-to-nearest-even, done by torch);
  * x ~ N(0, 1); gate weight std 1/sqrt(H) (logits of std ~1); expert and
    dense-MLP weights and biases std 0.02;
  * the Zipf-skewed workloads add a float32 gate bias b[e] = -s * ln(e + 1),
    the log of a Zipf(s) pmf up to a constant, so expert 0 is the hottest.

The shapes are those of the models on the pages: the 350M / 1.3B / 24B
+MoE-128 models ("[Review] DeepSpeed-MoE", section "MoE based NLG Model
Architecture"; "DeepSpeed-MoE Inference" wiki page, the model table in the
performance section) and the PR-MoE residual layer (same review, section
"PR-MoE: Pyramid-Residual-MoE").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

# tensor ids used in the per-tensor seed
TID_X, TID_GATE_W, TID_W1, TID_B1, TID_W2, TID_B2 = 0, 1, 2, 3, 4, 5
TID_MLP_W1, TID_MLP_B1, TID_MLP_W2, TID_MLP_B2 = 6, 7, 8, 9

WEIGHT_STD = 0.02

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class LayerShape:
    """One MoE FFN layer configuration (one GPU's share of it)."""
    name: str
    T: int                 # tokens in the batch
    H: int                 # hidden size
    F: int                 # expert FFN width
    E: int                 # gate width = number of global experts
    E_loc: int             # experts held by this GPU
    k: int                 # experts per token (1 or 2)
    cf: float              # capacity factor
    dtype: str             # "f32" | "f16" | "bf16"
    mlp_type: str = "standard"   # "standard" | "residual"
    zipf_s: Optional[float] = None
    e_lo: int = 0          # first local expert
    renorm: bool = False   # renormalise the top-k weights
    one_launch: bool = False  # decode path: both expert products in one launch

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @property
    def residual(self) -> bool:
        return self.mlp_type == "residual"

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


# The five workloads of the headline benchmark table.
WORKLOADS = {
    # tiny layer, fp32, the oracle finishes it instantly
    "tiny": LayerShape("tiny", T=256, H=64, F=256, E=8, E_loc=8, k=1, cf=1.0, dtype="f32"),
    # 350M+MoE-128 decode step: 8 tokens, weight-bandwidth bound
    "decode_350m_moe128": LayerShape("decode_350m_moe128", T=8, H=1024, F=4096, E=128,
                                     E_loc=128, k=1, cf=1.0, dtype="f16"),
    # 1.3B+MoE-128 prefill: Zipf(1.1) gate bias makes hot experts and drops
    "prefill_1p3b_moe128": LayerShape("prefill_1p3b_moe128", T=4096, H=2048, F=8192, E=128,
                                      E_loc=128, k=1, cf=1.25, dtype="f16", zipf_s=1.1),
    # PR-MoE residual layer: dense MLP + one routed expert of 64
    "prmoe_residual": LayerShape("prmoe_residual", T=2048, H=2048, F=8192, E=64, E_loc=64,
                                 k=1, cf=2.0, dtype="f16", mlp_type="residual"),
    # 24B+MoE-128: one GPU's share of 16 experts (0..15), top-2, Zipf(1.0)
    "share_24b_moe128": LayerShape("share_24b_moe128", T=16384, H=8192, F=32768, E=128,
                                   E_loc=16, k=2, cf=1.25, dtype="f16", zipf_s=1.0),
    # the same share at a decode step (8 tokens): expert rows of 16 / 64 KB, the
    # second product's K split over four waves in the decode kernels
    "decode_24b_share": LayerShape("decode_24b_share", T=8, H=8192, F=32768, E=128,
                                   E_loc=16, k=2, cf=1.0, dtype="f16", zipf_s=1.0),
}

# Reduced versions of the large workloads: same structure (k, cf, skew, mode,
# local share), sizes the fp64 oracle finishes in seconds while still spanning
# several GEMM tiles and ragged segment tails.
REDUCED = {
    "prefill_reduced": LayerShape("prefill_reduced", T=1024, H=512, F=1024, E=64, E_loc=64,
                                  k=1, cf=1.25, dtype="f16", zipf_s=1.1),
    "residual_reduced": LayerShape("residual_reduced", T=512, H=256, F=1024, E=16, E_loc=16,
                                   k=1, cf=2.0, dtype="f16", mlp_type="residual"),
    "share_reduced": LayerShape("share_reduced", T=2048, H=512, F=2048, E=32, E_loc=8,
                                k=2, cf=1.25, dtype="f16", zipf_s=1.0),
    "decode_reduced": LayerShape("decode_reduced", T=8, H=512, F=2048, E=64, E_loc=64,
                                 k=1, cf=1.0, dtype="f16"),
}


# Stacks of MoE layers run back to back, each layer's output feeding the next.
# Shape: the 1.3B model of the pages' inference example (hidden 2048, 24 layers;
# an MoE FFN every other layer gives 12 MoE layers), F = 4H, fp16.
#   * Top2-MoE and Residual-MoE at equal shapes (64 experts): the two ways of
#     giving each token two FFNs compared in the "Phenomenon2" part of the
#     review's PR-MoE section (top-2 routing vs a fixed MLP plus one routed expert);
#   * a PR-MoE pyramid: residual layers with more experts in the last layers
#     (the pages fix only "more experts in the last few layers"; read here as
#     32 experts in the first 10 MoE layers and 64 in the last 2).
def _stack(name: str, T: int, experts, k: int, mlp_type: str):
    return [LayerShape(f"{name}_l{i}", T=T, H=2048, F=8192, E=e, E_loc=e, k=k, cf=1.0, dtype="f16",
                       mlp_type=mlp_type) for i, e in enumerate(experts)]


_PYRAMID = [32] * 10 + [64] * 2
STACKS = {
    "top2_e64_decode": _stack("top2_e64_decode", 8, [64] * 12, 2, "standard"),
    "residual_e64_decode": _stack("residual_e64_decode", 8, [64] * 12, 1, "residual"),
    "prmoe_pyramid_decode": _stack("prmoe_pyramid_decode", 8, _PYRAMID, 1, "residual"),
    "top2_e64_prefill": _stack("top2_e64_prefill", 2048, [64] * 12, 2, "standard"),
    "residual_e64_prefill": _stack("residual_e64_prefill", 2048, [64] * 12, 1, "residual"),
    "prmoe_pyramid_prefill": _stack("prmoe_pyramid_prefill", 2048, _PYRAMID, 1, "residual"),
}

def _mix64(*vals: int) -> int:
    """splitmix64 over a tuple of ints -> a 63-bit torch seed."""
    z = 0x9E3779B97F4A7C15
    mask = (1 << 64) - 1
    for v in vals:
        z = (z + (v & mask) + 0x9E3779B97F4A7C15) & mask
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        z = z ^ (z >> 31)
    return z & ((1 << 63) - 1)


def _normal(shape, std: float, dtype: torch.dtype, device, seed: int, tid: int, expert: int = 0):
    g = torch.Generator(device=device)
    g.manual_seed(_mix64(seed, tid, expert))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def zipf_gate_bias(E: int, s: float, device="cpu") -> torch.Tensor:
    """b[e] = -s * ln(e + 1) in float32 (log Zipf(s) pmf up to a constant)."""
    return torch.tensor([-s * math.log(e + 1) for e in range(E)], dtype=torch.float32, device=device)


def make_x(shape: LayerShape, seed: int = 0, device="cpu") -> torch.Tensor:
    return _normal((shape.T, shape.H), 1.0, shape.torch_dtype, device, seed, TID_X)


def make_weights(shape: LayerShape, seed: int = 0, device="cpu") -> dict:
    """Gate, local-expert and (residual mode) dense-MLP weights, nn.Linear layout."""
    dt = shape.torch_dtype
    H, F, E = shape.H, shape.F, shape.E
    w = {
        "gate_w": _normal((E, H), 1.0 / math.sqrt(H), dt, device, seed, TID_GATE_W),
        "gate_b": zipf_gate_bias(E, shape.zipf_s, device) if shape.zipf_s is not None else None,
    }
    w1 = torch.empty((shape.E_loc, F, H), dtype=dt, device=device)
    b1 = torch.empty((shape.E_loc, F), dtype=dt, device=device)
    w2 = torch.empty((shape.E_loc, H, F), dtype=dt, device=device)
    b2 = torch.empty((shape.E_loc, H), dtype=dt, device=device)
    for i in range(shape.E_loc):
        e = shape.e_lo + i          # global expert index: a share sees the full layer's weights
        w1[i] = _normal((F, H), WEIGHT_STD, dt, device, seed, TID_W1, e)
        b1[i] = _normal((F,), WEIGHT_STD, dt, device, seed, TID_B1, e)
        w2[i] = _normal((H, F), WEIGHT_STD, dt, device, seed, TID_W2, e)
        b2[i] = _normal((H,), WEIGHT_STD, dt, device, seed, TID_B2, e)
    w.update(w1=w1, b1=b1, w2=w2, b2=b2)
    if shape.residual:
        w["mlp_w1"] = _normal((F, H), WEIGHT_STD, dt, device, seed, TID_MLP_W1)
        w["mlp_b1"] = _normal((F,), WEIGHT_STD, dt, device, seed, TID_MLP_B1)
        w["mlp_w2"] = _normal((H, F), WEIGHT_STD, dt, device, seed, TID_MLP_W2)
        w["mlp_b2"] = _normal((H,), WEIGHT_STD, dt, device, seed, TID_MLP_B2)
    return w


def to_host_f64_ready(t: Optional[torch.Tensor]):
    """A host numpy array holding exactly the tensor's values (bf16 widened to f32)."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()
