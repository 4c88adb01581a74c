"""Per-expert weight placement through the C ABI: pointer tables into device
memory, experts read straight from pinned host memory, and the expert store's
device cache after routing-driven updates (with evictions). The kernels do the
same arithmetic on the same values wherever the weights live, so every
placement must reproduce the contiguous-weights output bit for bit, and every
output is also compared with the fp64 oracle's layer on the same inputs (to
the tolerance of the I/O dtype); the residency the store picks is checked
against the demand it was given."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_transformer_moe_amd import binding as B
from mixture_experts_transformer_moe_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

CASES = {
    # streaming expert kernels (8 tokens, routing inside the first kernel)
    "decode": W.LayerShape("store_dec", T=8, H=512, F=1024, E=32, E_loc=32, k=2, cf=1.0, dtype="f16"),
    # grouped GEMM (segments of up to 64 rows), a share of the experts
    "gemm": W.LayerShape("store_gemm", T=512, H=256, F=512, E=16, E_loc=8, e_lo=4, k=2, cf=1.0, dtype="f16"),
    # eight-wave ping-pong tiles (160 x 256, direct-to-LDS loads) reading each
    # expert's weights through the pointer tables
    "gemm_pingpong": W.LayerShape("store_pp", T=1024, H=512, F=1024, E=8, E_loc=8, k=2, cf=1.25, dtype="f16"),
}


def _oracle_y(shape, L, x, w):
    """The oracle's layer output on host copies of the same inputs, the GPU's
    choice adopted for near-tie tokens (routing must match everywhere else)."""
    idx = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    B.moe_gate(L.desc, x, L.weights["gate_w"], L.weights["gate_b"], idx, tw, None, L.ws)
    torch.cuda.synchronize()
    hx, hw = G.host(x), G.host_weights({k: v for k, v in w.items() if v is not None})
    hw.setdefault("gate_b", None)
    route = oracle.route(hx, hw["gate_w"], hw["gate_b"], shape.k, shape.renorm)
    override = G.adopt_near_ties(route, G.host(idx), shape.k)
    return oracle.layer_forward(hx, hw, E=shape.E, k=shape.k, cf=shape.cf, e_lo=shape.e_lo, E_loc=shape.E_loc,
                                residual=shape.residual, renorm=shape.renorm, override=override)["y"]


def _check(y, ref, y_oracle, shape, what):
    """Bit-exact against the contiguous-weights output, and within the dtype's
    tolerance of the oracle."""
    assert torch.equal(y, ref), what
    G.assert_close(G.host(y), y_oracle, shape.dtype, what)


def _demand(shape, L, x):
    idx = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    demand = torch.empty(shape.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(shape.E_loc + 1, dtype=torch.int32, device="cuda")
    R = max(B.moe_max_rows(L.desc), 1)
    st = torch.empty(R, dtype=torch.int32, device="cuda")
    ts = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    B.moe_gate(L.desc, x, L.weights["gate_w"], L.weights["gate_b"], idx, tw, None, L.ws)
    B.moe_dispatch(L.desc, idx, x, demand, offsets, st, ts, None, L.ws)
    return demand.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_tables_into_device_weights(name):
    shape = CASES[name]
    G.say(f"[tables {name}] E_loc={shape.E_loc} T={shape.T}")
    x, w = G.device_case(shape, seed=2)
    plain = B.MoELayer(shape, w)
    ref = plain.forward(x)
    y_oracle = _oracle_y(shape, plain, x, w)
    tabs = {}
    for key in ("w1", "b1", "w2", "b2"):
        t = w[key]
        stride = t[0].numel() * t.element_size()
        tabs[key + "_experts"] = torch.tensor([t.data_ptr() + i * stride for i in range(shape.E_loc)],
                                              dtype=torch.int64, device="cuda")
    w2 = dict(w)
    w2.update(tabs)
    w2.update(w1=None, b1=None, w2=None, b2=None)
    y = B.MoELayer(shape, w2).forward(x)
    torch.cuda.synchronize()
    _check(y, ref, y_oracle, shape, f"{name}: pointer tables into device weights")


@pytest.mark.parametrize("name", list(CASES))
def test_store_host_reads_and_cache_updates(name):
    shape = CASES[name]
    x, w = G.device_case(shape, seed=3)
    plain = B.MoELayer(shape, w)
    ref = plain.forward(x)
    torch.cuda.synchronize()
    y_oracle = _oracle_y(shape, plain, x, w)
    slots = shape.E_loc // 4
    store = B.ExpertStore(shape, slots)
    try:
        store.fill({k: w[k].cpu() for k in ("w1", "b1", "w2", "b2")})
        L = B.MoELayer(shape, w, store=store)
        G.say(f"[store {name}] all experts host-resident")
        y0 = L.forward(x)
        torch.cuda.synchronize()
        _check(y0, ref, y_oracle, shape, f"{name}: all experts host-resident")
        assert np.all(store.residency() == -1)

        demand = _demand(shape, plain, x)
        local = demand[shape.e_lo:shape.e_lo + shape.E_loc]
        n = store.update(demand)
        res = store.residency()
        cached = set(np.nonzero(res >= 0)[0].tolist())
        want = [e for e in sorted(range(shape.E_loc), key=lambda e: (-local[e], e)) if local[e] > 0][:slots]
        G.say(f"  update 1: copied {n}, cached {sorted(cached)}, wanted {sorted(want)}")
        assert cached == set(want) and n == len(want)
        assert len(set(res[res >= 0].tolist())) == len(cached)          # distinct slots
        y1 = L.forward(x)
        torch.cuda.synchronize()
        _check(y1, ref, y_oracle, shape, f"{name}: after update 1")

        # demand moves to experts that are not cached: scores halve, the new ones win
        d2 = np.zeros(shape.E, dtype=np.int32)
        fresh = [e for e in range(shape.E_loc) if e not in cached][:slots]
        for e in fresh:
            d2[shape.e_lo + e] = 10 * int(local.max() + 1)
        n2 = store.update(d2)
        res2 = store.residency()
        G.say(f"  update 2: copied {n2}, cached {sorted(np.nonzero(res2 >= 0)[0].tolist())}")
        assert set(np.nonzero(res2 >= 0)[0].tolist()) == set(fresh) and n2 == len(fresh)
        y2 = L.forward(x)
        torch.cuda.synchronize()
        _check(y2, ref, y_oracle, shape, f"{name}: after update 2 (evictions)")
        # the same demand again changes nothing
        assert store.update(d2) == 0
        y3 = L.forward(x)
        torch.cuda.synchronize()
        _check(y3, ref, y_oracle, shape, f"{name}: unchanged update")
    finally:
        store.close()


@pytest.mark.parametrize("name", list(CASES))
def test_store_async_copies_on_a_second_stream(name):
    """Copies on a copy stream overlap with layers enqueued on the compute stream:
    before the commit those layers read the incoming experts from host memory,
    after it from their slots; either way the output is the contiguous-weights
    output bit for bit."""
    shape = CASES[name]
    x, w = G.device_case(shape, seed=5)
    plain = B.MoELayer(shape, w)
    ref = plain.forward(x)
    torch.cuda.synchronize()
    y_oracle = _oracle_y(shape, plain, x, w)
    slots = shape.E_loc // 4
    store = B.ExpertStore(shape, slots)
    copy = torch.cuda.Stream()          # default priority, like the compute stream
    try:
        store.fill({k: w[k].cpu() for k in ("w1", "b1", "w2", "b2")})
        L = B.MoELayer(shape, w, store=store)
        demand = _demand(shape, plain, x)
        local = demand[shape.e_lo:shape.e_lo + shape.E_loc]
        want = [e for e in sorted(range(shape.E_loc), key=lambda e: (-local[e], e)) if local[e] > 0][:slots]
        n = store.update_async(demand, copy)
        y_before = L.forward(x)          # enqueued while the copies may still run
        store.commit()
        y_after = L.forward(x)
        torch.cuda.synchronize()
        cached = set(np.nonzero(store.residency() >= 0)[0].tolist())
        G.say(f"[store async {name}] copied {n} on the copy stream, cached {sorted(cached)}")
        assert n == len(want) and cached == set(want)
        _check(y_before, ref, y_oracle, shape, f"{name}: async, before the commit")
        _check(y_after, ref, y_oracle, shape, f"{name}: async, after the commit")

        # evictions and new copies; a synchronous update commits the pending one first
        d2 = np.zeros(shape.E, dtype=np.int32)
        fresh = [e for e in range(shape.E_loc) if e not in cached][:slots]
        for e in fresh:
            d2[shape.e_lo + e] = 10 * int(local.max() + 1)
        n2 = store.update_async(d2, copy)
        y_mid = L.forward(x)
        assert store.update(d2) == 0
        y_end = L.forward(x)
        torch.cuda.synchronize()
        G.say(f"  second update: copied {n2}, cached {sorted(np.nonzero(store.residency() >= 0)[0].tolist())}")
        assert n2 == len(fresh) and set(np.nonzero(store.residency() >= 0)[0].tolist()) == set(fresh)
        _check(y_mid, ref, y_oracle, shape, f"{name}: second async update, before its commit")
        _check(y_end, ref, y_oracle, shape, f"{name}: after the synchronous update")
        with pytest.raises(B.MoeError):
            store.update_async(d2, torch.cuda.current_stream())   # the copy stream must be another stream
    finally:
        torch.cuda.synchronize()
        store.close()
