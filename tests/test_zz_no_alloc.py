"""moe_layer_forward_noalloc (the entry point that allocates nothing: the
library's own device scratch array replaces the workspace) against
moe_layer_forward with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller layer, each bit-identical to the workspace
entry point's output (same kernels, same arithmetic) and within the dtype's
tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_transformer_moe_amd import binding as B
from mixture_experts_transformer_moe_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _oracle_y(shape, x, w, L):
    idx = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    B.moe_gate(L.desc, x, w["gate_w"], w["gate_b"], idx, tw, None, L.ws)
    torch.cuda.synchronize()
    hx, hw = G.host(x), G.host_weights(w)
    route = oracle.route(hx, hw["gate_w"], hw["gate_b"], shape.k, shape.renorm)
    override = G.adopt_near_ties(route, G.host(idx), shape.k)
    return oracle.layer_forward(hx, hw, E=shape.E, k=shape.k, cf=shape.cf, e_lo=shape.e_lo, E_loc=shape.E_loc,
                                residual=shape.residual, renorm=shape.renorm, override=override)["y"]


def _run(shape, seed):
    x, w = G.device_case(shape, seed=seed)
    L = B.MoELayer(shape, w)
    ref = L.forward(x)
    y = torch.full_like(x, float("nan"))
    B.moe_layer_forward_noalloc(L.desc, L.cw, x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref), f"{shape.name}: no-allocation output differs from the workspace entry point's"
    G.assert_close(G.host(y), _oracle_y(shape, x, w, L), shape.dtype, f"{shape.name} (no allocation)")


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    big = W.REDUCED["share_reduced"]                   # grouped GEMM path, top-2 share, 7.8 MiB of scratch
    small = W.REDUCED["decode_reduced"]                 # streaming decode path, 50 KiB
    G.say(f"[noalloc] {big.name} then {small.name}")
    _run(big, seed=11)
    _run(small, seed=12)


def test_noalloc_largest_benchmark_layer_that_fits_then_decode():
    big = W.WORKLOADS["prefill_1p3b_moe128"]           # 104 MiB of the 128 MiB array
    assert B.moe_workspace_size(B.desc_from_shape(big)) <= B.NOALLOC_SCRATCH_BYTES
    G.say(f"[noalloc] {big.name} then decode_350m_moe128")
    x, w = G.device_case(big, seed=0)
    L = B.MoELayer(big, w)
    ref = L.forward(x)
    y = torch.empty_like(x)
    B.moe_layer_forward_noalloc(L.desc, L.cw, x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    del x, w, L, ref, y
    torch.cuda.empty_cache()
    _run(W.WORKLOADS["decode_350m_moe128"], seed=3)


def test_noalloc_refuses_layers_beyond_its_scratch():
    d = B.desc_from_shape(W.WORKLOADS["share_24b_moe128"])   # 497 MiB of workspace
    x = torch.empty((16, 16), dtype=torch.float16, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_forward_noalloc(d, B.LayerWeights(), x, x)
    assert e.value.status == B.MOE_ERR_WORKSPACE_TOO_SMALL
