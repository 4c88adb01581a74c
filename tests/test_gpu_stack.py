"""Stacks of MoE layers chained through the C ABI: layer l reads layer l - 1's
output, as the layer-stack benchmark runs them. Every layer is compared with the
fp64 oracle fed the same (GPU-produced) input, so the test covers the chaining
(buffers, stream order, per-layer workspaces) and each layer type in the stack:
residual layers with different expert counts (a PR-MoE pyramid) and a top-2
layer, on the grouped-GEMM path and on the decode path."""
import pytest
import torch

import oracle
from mixture_experts_transformer_moe_amd import binding as B
from mixture_experts_transformer_moe_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _stack(T, H, F, experts_modes):
    return [W.LayerShape(f"stack_{T}_{i}", T=T, H=H, F=F, E=e, E_loc=e, k=k, cf=1.0, dtype="f16", mlp_type=m)
            for i, (e, k, m) in enumerate(experts_modes)]


STACKS = {
    # segments of up to 32-64 rows: grouped GEMM path
    "gemm": _stack(256, 256, 512, [(8, 1, "residual"), (16, 1, "residual"), (16, 2, "standard")]),
    # 8 tokens: streaming expert kernels, routing inside the first one, dense MLP on the decode path
    "decode": _stack(8, 512, 1024, [(32, 1, "residual"), (64, 1, "residual"), (64, 2, "standard")]),
}


@pytest.mark.parametrize("name", list(STACKS))
def test_stack_layers_match_oracle(name):
    shapes = STACKS[name]
    G.say(f"[stack {name}] " + ", ".join(f"E={s.E} k={s.k} {s.mlp_type}" for s in shapes))
    layers = [B.MoELayer(sh, W.make_weights(sh, seed=10 + i, device="cuda")) for i, sh in enumerate(shapes)]
    x = W.make_x(shapes[0], seed=3, device="cuda")
    io = []
    cur = x
    for L in layers:
        y = torch.empty_like(cur)
        L.forward(cur, y)
        io.append((cur, y))
        cur = y
    torch.cuda.synchronize()
    for L, (xin, y) in zip(layers, io):
        sh = L.shape
        hx, hw = G.host(xin), G.host_weights(L.weights)
        idx = torch.empty((sh.T, sh.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((sh.T, sh.k), dtype=torch.float32, device="cuda")
        B.moe_gate(L.desc, xin, L.weights["gate_w"], L.weights["gate_b"], idx, tw, None, L.ws)
        torch.cuda.synchronize()
        route = oracle.route(hx, hw["gate_w"], hw["gate_b"], sh.k, sh.renorm)
        override = G.adopt_near_ties(route, G.host(idx), sh.k)
        ref = oracle.layer_forward(hx, hw, E=sh.E, k=sh.k, cf=sh.cf, e_lo=sh.e_lo, E_loc=sh.E_loc,
                                   residual=sh.residual, renorm=sh.renorm, override=override)
        G.assert_close(G.host(y), ref["y"], sh.dtype, f"layer {sh.name} (near ties adopted: {len(override)})")

