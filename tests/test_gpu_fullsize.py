"""The benchmark layers at full size (needs a GPU): routing and dispatch compared
with the oracle on every token (bit-exact after near-tie adoption), outputs on a
seeded sample of tokens computed one by one by the oracle, and every fully
dropped token's output row checked to be exactly zero."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_transformer_moe_amd import binding as B
from mixture_experts_transformer_moe_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _routing_on_gpu(shape, x, w):
    desc = B.desc_from_shape(shape)
    T, k, E = shape.T, shape.k, shape.E
    R_max = B.moe_max_rows(desc)
    ws = torch.empty(max(B.moe_workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    demand = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(shape.E_loc + 1, dtype=torch.int32, device="cuda")
    slot_token = torch.empty(R_max, dtype=torch.int32, device="cuda")
    token_slot = torch.empty((T, k), dtype=torch.int32, device="cuda")
    B.moe_gate(desc, x, w["gate_w"], w["gate_b"], idx, tw, None, ws)
    B.moe_dispatch(desc, idx, x, demand, offsets, slot_token, token_slot, None, ws)
    torch.cuda.synchronize()
    del ws
    return {n: G.host(v) for n, v in dict(idx=idx, w=tw, demand=demand, offsets=offsets, slot_token=slot_token,
                                            token_slot=token_slot).items()}


def _pick_tokens(token_slot, slot_expert, T, n_max=48, max_experts=4, seed=0):
    """Seeded sample: tokens whose kept experts stay within a few experts (so the
    oracle needs only those experts' weights), plus fully dropped tokens."""
    rng = np.random.default_rng(seed)
    chosen, experts = [], set()
    order = np.concatenate([[0, T - 1], rng.permutation(T)])
    for t in order:
        t = int(t)
        if t in chosen:
            continue
        es = {int(slot_expert[s]) for s in token_slot[t] if s >= 0}
        if len(experts | es) <= max_experts:
            chosen.append(t)
            experts |= es
        if len(chosen) >= n_max:
            break
    return np.array(sorted(chosen)), sorted(experts)


@pytest.mark.parametrize("name", ["prefill_1p3b_moe128", "prmoe_residual", "share_24b_moe128"])
def test_fullsize_layer(name):
    shape = W.WORKLOADS[name]
    G.say(f"[full {name}] T={shape.T} H={shape.H} F={shape.F} E={shape.E} E_loc={shape.E_loc} k={shape.k}")
    x, w = G.device_case(shape, seed=0)
    y = B.MoELayer(shape, w).forward(x)
    torch.cuda.synchronize()
    g = _routing_on_gpu(shape, x, w)
    hx = G.host(x)
    gw = G.host(w["gate_w"])
    gb = G.host(w["gate_b"]) if w["gate_b"] is not None else None
    route = oracle.route(hx, gw, gb, shape.k, shape.renorm)
    override = G.adopt_near_ties(route, g["idx"], shape.k)
    G.say(f"  near-tie tokens adopted: {len(override)} of {shape.T}")
    route = oracle.route(hx, gw, gb, shape.k, shape.renorm, override=override)
    C = oracle.capacity(shape.T, shape.E, shape.k, shape.cf)
    d = oracle.dispatch(route["idx"], shape.E, C, shape.e_lo, shape.E_loc)
    assert np.array_equal(g["demand"], d["demand"])
    assert np.array_equal(g["offsets"], d["offsets"])
    assert np.array_equal(g["token_slot"], d["token_slot"])
    assert np.array_equal(g["slot_token"][: d["R"]], d["slot_token"])
    assert np.max(np.abs(g["w"] - route["w"])) < 2e-5
    G.say(f"  C={C} rows={d['R']} active={int((np.diff(d['offsets']) > 0).sum())} "
          f"dropped assignments={int((d['token_slot'] < 0).sum())}")

    yh = G.host(y)
    slot_expert = np.repeat(np.arange(shape.E_loc), np.diff(d["offsets"]))
    if not shape.residual:
        none_kept = np.all(d["token_slot"] < 0, axis=1)
        assert np.all(yh[none_kept] == 0), "tokens with nothing kept must get exactly zero"
    toks, experts = _pick_tokens(d["token_slot"], slot_expert, shape.T)
    G.say(f"  sampled {len(toks)} tokens over experts {experts}")
    ew = {e: (G.host(w["w1"][e]), G.host(w["b1"][e]), G.host(w["w2"][e]), G.host(w["b2"][e])) for e in experts}
    dense = None
    if shape.residual:
        dense = (G.host(w["mlp_w1"]), G.host(w["mlp_b1"]), G.host(w["mlp_w2"]), G.host(w["mlp_b2"]))
    ref = oracle.layer_rows(hx[toks], d["token_slot"][toks], route["w"][toks], slot_expert, ew, dense)
    G.assert_close(yh[toks], ref, shape.dtype, f"{name} sampled rows")
    del x, w, y
    torch.cuda.empty_cache()
