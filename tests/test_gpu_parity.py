"""HIP path vs the fp64 oracle, element by element, through the C ABI (needs a GPU).

Sizes here are ones the oracle finishes in seconds while spanning several GEMM
tiles and ragged segment tails; the full benchmark shapes are covered by
test_gpu_fullsize.py on sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_transformer_moe_amd import binding as B
from mixture_experts_transformer_moe_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

R = W.REDUCED
CASES = {
    "tiny_f32": W.WORKLOADS["tiny"],
    "decode_reduced": R["decode_reduced"],
    "decode_full_350m": W.WORKLOADS["decode_350m_moe128"],
    "prefill_reduced": R["prefill_reduced"],
    "residual_reduced": R["residual_reduced"],
    "share_reduced_lo": R["share_reduced"],
    "share_reduced_hi": R["share_reduced"].with_(e_lo=24),
    "share_reduced_bf16": R["share_reduced"].with_(dtype="bf16"),
    "decode_reduced_bf16": R["decode_reduced"].with_(dtype="bf16"),
    "share_reduced_renorm": R["share_reduced"].with_(renorm=True, name="share_renorm"),
    "decode_t1": R["decode_reduced"].with_(T=1),
    "decode_c4": R["decode_reduced"].with_(T=64, cf=4.0),          # segments of up to 4 rows
    "residual_decode": R["residual_reduced"].with_(T=8, H=512, F=1024),
    "k2_e2": W.LayerShape("k2_e2", T=200, H=128, F=256, E=2, E_loc=2, k=2, cf=0.75, dtype="f16"),
    "e1_dense": W.LayerShape("e1", T=100, H=64, F=192, E=1, E_loc=1, k=1, cf=1.0, dtype="f16"),
    "gemm_mid_rows": W.LayerShape("mid", T=600, H=256, F=512, E=8, E_loc=8, k=2, cf=1.0, dtype="f16"),
    "decode_f32_h512": W.LayerShape("dec32", T=8, H=512, F=512, E=32, E_loc=32, k=1, cf=1.0, dtype="f32"),
    "decode_f32_h256_k2": W.LayerShape("dec32b", T=5, H=256, F=256, E=16, E_loc=16, k=2, cf=2.0, dtype="f32"),
    "decode_k2_share": W.LayerShape("deck2", T=8, H=1024, F=2048, E=64, E_loc=16, e_lo=16, k=2, cf=1.0,
                                    dtype="f16"),
    # grouped GEMM with two stages in flight (tiles of <= 64 rows): 64-wide column
    # tiles (H = 320), bf16, and full 64-row tiles with top-2
    # second GEMM with long weight rows (F = 8192): 64-column tiles by the plan
    "gemm_long_f_bn64": W.LayerShape("glf", T=512, H=256, F=8192, E=16, E_loc=16, k=1, cf=1.25, dtype="f16"),
    "gemm_bn64": W.LayerShape("gbn64", T=256, H=320, F=512, E=16, E_loc=16, k=1, cf=1.0, dtype="f16"),
    "gemm_bf16_bm32": W.LayerShape("gbf", T=512, H=512, F=1024, E=16, E_loc=16, k=1, cf=1.0, dtype="bf16"),
    "gemm_bm64_k2": W.LayerShape("gk2", T=512, H=512, F=768, E=32, E_loc=32, k=2, cf=2.0, dtype="f16"),
    # eight-wave 320 x 256 tiles: segments of up to C = 320 rows, one m-tile each
    "gemm_bm320": W.LayerShape("g160", T=1024, H=512, F=1024, E=8, E_loc=8, k=2, cf=1.25, dtype="f16"),
    "gemm_bm320_bf16_share": W.LayerShape("g160b", T=1024, H=512, F=1024, E=8, E_loc=4, e_lo=2, k=2, cf=1.25,
                                          dtype="bf16"),
    # 320 x 256 tiles with the dense MLP's tiles in the same launches: expert
    # weights streamed, the MLP's cached (two copies of the K loop)
    "residual_bm320": W.LayerShape("r160", T=1024, H=512, F=1024, E=4, E_loc=4, k=1, cf=1.25, dtype="f16",
                                   mlp_type="residual"),
    # 128 x 256 ping-pong tiles with the dense MLP's tiles in the same launches;
    # 256 x 256 tiles in bf16 with top-2 (segments of up to C = 150 rows); the
    # folded combine on 128 x 256 tiles (C = 128)
    "residual_bm128": W.LayerShape("r128", T=1024, H=512, F=1024, E=8, E_loc=8, k=1, cf=1.0, dtype="f16",
                                   mlp_type="residual"),
    "gemm_bm256_bf16_k2": W.LayerShape("g128b", T=600, H=256, F=512, E=8, E_loc=8, k=2, cf=1.0, dtype="bf16"),
    "gemm_bm128_fold": W.LayerShape("g128f", T=1024, H=256, F=512, E=8, E_loc=8, k=1, cf=1.0, dtype="f16"),
    # 320 x 256 tiles over a batch of fewer than 320 tokens (C = 300, segments of
    # 150 rows): every activation load of the first GEMM must stay inside x's
    # 150 rows
    "gemm_bm320_t150": W.LayerShape("g160t", T=150, H=256, F=512, E=2, E_loc=2, k=2, cf=2.0, dtype="f16"),
    # ping-pong tiles at widths that are multiples of 256 but not of 512: 320 x
    # 256 tiles of a 768-wide first product, and a residual layer with both
    # products and the dense MLP on 128 x 256 tiles (H = F = 768, bf16)
    "gemm_bm320_f768": W.LayerShape("g160n", T=1024, H=512, F=768, E=8, E_loc=8, k=2, cf=1.25, dtype="f16"),
    "residual_bm128_bn256": W.LayerShape("r128n", T=1024, H=768, F=768, E=8, E_loc=8, k=1, cf=1.0, dtype="bf16",
                                         mlp_type="residual"),
    # edge cases: the maximum expert count (8 logits per lane in the top-k), a
    # ragged token count (gate token blocks of 8), heavy drops (cf = 0.1), one
    # token through a residual layer, and a share of a single local expert
    # top-1 layer of 320-row segments: the folded combine on the 320 x 256 tiles
    "gemm_bm320_fold": W.LayerShape("g320f", T=2048, H=256, F=512, E=8, E_loc=8, k=1, cf=1.25, dtype="f16"),
    # top-1 layers whose combine runs in the second GEMM's epilogue on the
    # ping-pong tiles (segments > 64 rows), one with non-local tokens to zero
    "gemm_pp_fold": W.LayerShape("gppf", T=2048, H=256, F=512, E=8, E_loc=8, k=1, cf=1.0, dtype="f16"),
    "gemm_pp_fold_share_bf16": W.LayerShape("gppfs", T=1500, H=512, F=768, E=8, E_loc=3, e_lo=4, k=1, cf=1.25,
                                            dtype="bf16"),
    # one local expert of 64: four tiles in the first GEMM, whose work-groups zero
    # ~1000 dropped / non-local tokens' rows each
    "gemm_fold_few_tiles": W.LayerShape("gfft", T=4096, H=256, F=512, E=64, E_loc=1, k=1, cf=1.0, dtype="f16"),
    # decode kernels with K split over 2 / 4 waves (K = 16384 / 32768): the second
    # product (long F), the first (long H), top-2 in bf16, and a residual layer
    # whose dense MLP runs on the decode kernels
    "decode_ksplit2_f": W.LayerShape("dk2f", T=8, H=512, F=16384, E=16, E_loc=16, k=1, cf=1.0, dtype="f16"),
    "decode_ksplit4_f_k2_bf16": W.LayerShape("dk4f", T=4, H=1024, F=32768, E=4, E_loc=4, k=2, cf=2.0,
                                             dtype="bf16"),
    "decode_ksplit2_h": W.LayerShape("dk2h", T=8, H=16384, F=512, E=16, E_loc=16, k=1, cf=1.0, dtype="f16"),
    "decode_ksplit4_h": W.LayerShape("dk4h", T=2, H=32768, F=1024, E=4, E_loc=4, k=1, cf=2.0, dtype="f16"),
    "residual_decode_ksplit": W.LayerShape("rdk", T=4, H=512, F=16384, E=8, E_loc=8, k=1, cf=1.0, dtype="f16",
                                           mlp_type="residual"),
    "e512_decode": W.LayerShape("e512d", T=8, H=512, F=512, E=512, E_loc=512, k=2, cf=1.0, dtype="f16"),
    "e512_gemm": W.LayerShape("e512g", T=600, H=256, F=512, E=512, E_loc=512, k=1, cf=4.0, dtype="f16"),
    "ragged_t13": W.LayerShape("t13", T=13, H=512, F=1024, E=16, E_loc=16, k=2, cf=1.0, dtype="f16"),
    "heavy_drop": W.LayerShape("drop", T=1000, H=256, F=512, E=8, E_loc=8, k=2, cf=0.1, dtype="f16"),
    "residual_t1": W.LayerShape("rt1", T=1, H=512, F=1024, E=8, E_loc=8, k=1, cf=1.0, dtype="f16",
                                mlp_type="residual"),
    "share_eloc1": W.LayerShape("el1", T=256, H=256, F=512, E=16, E_loc=1, e_lo=5, k=2, cf=1.0, dtype="bf16"),
    # residual pass-through: a share of 2 of 16 experts (most rows are MLP(x)
    # alone), and heavy drops (C = 4 of 600 tokens per expert: decode expert
    # kernels beside the dense MLP's GEMMs)
    "residual_share_passthrough": W.LayerShape("rsp", T=512, H=256, F=512, E=16, E_loc=2, e_lo=3, k=1, cf=1.0,
                                               dtype="f16", mlp_type="residual"),
    "residual_heavy_drop": W.LayerShape("rhd", T=600, H=256, F=512, E=8, E_loc=8, k=1, cf=0.05, dtype="f16",
                                        mlp_type="residual"),
    # the dense MLP in launches of its own on the ping-pong kernel's single-
    # segment tiles (128 x 256, no tile list), beside 16-row expert tiles
    "residual_dense_pingpong": W.LayerShape("rdp", T=4096, H=256, F=4096, E=16, E_loc=16, k=1, cf=0.03125,
                                            dtype="f16", mlp_type="residual"),
    # streaming expert kernels fed by the dispatch kernel (batch too large to route in-kernel)
    "decode_unrouted": W.LayerShape("decun", T=512, H=512, F=512, E=256, E_loc=256, k=1, cf=1.0, dtype="f16"),
    # the multi-block dispatch writing the GEMM tile lists from its scan block:
    # sixteen dispatch blocks with one expert, and eighteen with 32 experts, top-2
    "gemm_multi_e8": W.LayerShape("gm8", T=16384, H=64, F=128, E=8, E_loc=8, k=1, cf=1.0, dtype="f16"),
    "gemm_multi_block": W.LayerShape("gmb", T=9000, H=128, F=256, E=32, E_loc=32, k=2, cf=1.0, dtype="f16"),
    # matrix-core gate with K in four slices (H = 2048: 32 steps of 128 bytes),
    # fp32 partial logits summed by the softmax / top-k, probabilities included
    "gate_k_slices": W.LayerShape("gks", T=512, H=2048, F=256, E=64, E_loc=8, e_lo=8, k=2, cf=1.0, dtype="f16"),
    "gate_k_slices_bf16": W.LayerShape("gksb", T=300, H=1024, F=256, E=128, E_loc=16, k=1, cf=1.0, dtype="bf16"),
    # softmax / top-k and the multi-block dispatch in one launch (matrix-core
    # gate, more than 1024 assignments): top-2 with a ragged last ranker block
    "route_one_launch_k2": W.LayerShape("rk2", T=3000, H=256, F=512, E=64, E_loc=64, k=2, cf=1.0, dtype="f16"),
    # ... a share of 16 of 128 Zipf-skewed experts, combine folded, bf16
    "route_one_launch_share": W.LayerShape("rsh", T=2500, H=512, F=256, E=128, E_loc=16, e_lo=40, k=1, cf=1.25,
                                           dtype="bf16", zipf_s=1.1),
    # ... the gate's K in four slices (partial logits added in the launch)
    "route_one_launch_kslices": W.LayerShape("rks", T=2100, H=2048, F=256, E=64, E_loc=64, k=1, cf=1.0, dtype="f16"),
    # ... the most ranker blocks it takes (64 blocks of 1024 assignments)
    "route_one_launch_64_blocks": W.LayerShape("r64", T=32768, H=64, F=128, E=64, E_loc=64, k=2, cf=1.0, dtype="f16"),
    # ... a residual layer (the dense MLP's tiles in the tile lists it writes)
    "route_one_launch_residual": W.LayerShape("rres", T=2048, H=256, F=512, E=64, E_loc=64, k=1, cf=2.0, dtype="f16",
                                              mlp_type="residual"),
    # ... feeding the streaming expert kernels (no tile lists: a ranker writes the offsets)
    "route_one_launch_stream": W.LayerShape("rstr", T=1100, H=512, F=512, E=256, E_loc=256, k=1, cf=1.0, dtype="f16"),
    # ... two ranker blocks, the second holding one assignment
    "route_one_launch_1025": W.LayerShape("r1025", T=1025, H=256, F=512, E=64, E_loc=64, k=1, cf=1.0, dtype="f16"),
    # ... the largest expert count (two threads per expert add the block counts)
    "route_one_launch_e512": W.LayerShape("r512", T=1500, H=256, F=512, E=512, E_loc=512, k=1, cf=4.0, dtype="f16"),
}


def _oracle_full(shape, hx, hw, override):
    return oracle.layer_forward(hx, hw, E=shape.E, k=shape.k, cf=shape.cf, e_lo=shape.e_lo, E_loc=shape.E_loc,
                                residual=shape.residual, renorm=shape.renorm, override=override)


@pytest.mark.parametrize("name", list(CASES))
def test_steps_and_layer_match_oracle(name):
    shape = CASES[name]
    G.say(f"[case {name}] T={shape.T} H={shape.H} F={shape.F} E={shape.E} E_loc={shape.E_loc} "
          f"k={shape.k} cf={shape.cf} {shape.dtype} {shape.mlp_type}")
    x, w = G.device_case(shape, seed=0)
    g = G.gpu_steps(shape, x, w)
    hx, hw = G.host(x), G.host_weights(w)

    # gate: routing bit-exact except near-ties, which must be legal and are adopted
    route = oracle.route(hx, hw["gate_w"], hw["gate_b"], shape.k, shape.renorm)
    override = G.adopt_near_ties(route, g["idx"], shape.k)
    G.say(f"  near-tie tokens adopted: {len(override)}")
    ref = _oracle_full(shape, hx, hw, override)
    assert np.max(np.abs(g["probs"] - ref["p"])) < 2e-5
    assert np.allclose(g["probs"].sum(1), 1.0, atol=1e-5)
    assert np.max(np.abs(g["w"] - ref["w"])) < 2e-5

    # dispatch: bit-exact
    assert np.array_equal(g["demand"], ref["demand"])
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["token_slot"], ref["token_slot"])
    assert g["R"] == ref["R"]
    assert np.array_equal(g["slot_token"][: ref["R"]], ref["slot_token"])
    assert np.all(g["slot_token"][ref["R"]:] == -1)
    assert np.array_equal(g["x_disp"][: ref["R"]], hx[ref["slot_token"]])
    assert np.all(g["x_disp"][ref["R"]:] == 0)

    # expert FFN and dense MLP before the combine (fp32 outputs, I/O-dtype inputs)
    if ref["R"]:
        G.assert_close(g["y_disp"], ref["y_disp"], shape.dtype, "expert ffn rows")
    if shape.residual:
        G.assert_close(g["dense"], ref["dense"], shape.dtype, "dense mlp")
    G.assert_close(g["y"], ref["y"], shape.dtype, "combined output (step calls)")

    # the fused layer entry point gives the same bits as the step chain
    layer = B.MoELayer(shape, w)
    y = layer.forward(x)
    torch.cuda.synchronize()
    assert np.array_equal(G.host(y), g["y"]), "moe_layer_forward differs from the step chain"
    G.assert_close(G.host(y), ref["y"], shape.dtype, "moe_layer_forward")
    # reruns are bit-identical (no atomics)
    y2 = layer.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("T,E,k,E_loc,e_lo,cf,hot", [
    (100, 16, 2, 16, 0, 1.0, False),      # one-block path
    (3000, 16, 2, 16, 0, 1.0, True),      # multi-block path, hot expert
    (3000, 64, 1, 8, 40, 1.25, True),     # local share
    (777, 5, 2, 3, 1, 0.5, False),
    (1024, 8, 1, 8, 0, 1.0, True),        # exactly one block
    (1025, 8, 1, 8, 0, 1.0, True),        # one block plus one assignment
    (5000, 512, 2, 512, 0, 1.0, False),   # multi-block with the largest expert count
    (16385, 8, 1, 8, 0, 1.0, True),       # seventeen blocks, the last holding one assignment
    (9000, 32, 2, 24, 4, 1.0, False),     # multi-block, local share, top-2
    (4096, 64, 2, 64, 0, 1.0, True),      # eight blocks, top-2, hot expert
    (8193, 8, 1, 8, 0, 1.0, False),       # nine blocks, the last holding one assignment
    (2500, 128, 1, 16, 100, 1.25, True),  # local share near the top of the expert range
])
def test_dispatch_fed_oracle_routing(T, E, k, E_loc, e_lo, cf, hot):
    G.say(f"[dispatch] T={T} E={E} k={k} E_loc={E_loc} e_lo={e_lo} cf={cf} hot={hot}")
    rng = np.random.default_rng(T * 31 + E)
    z = rng.standard_normal((T, E))
    if hot:
        z[:, 0] += 2.0
    idx, _ = oracle.top_k(z, k)
    C = oracle.capacity(T, E, k, cf)
    ref = oracle.dispatch(idx, E, C, e_lo, E_loc)
    shape = W.LayerShape("disp", T=T, H=64, F=64, E=E, E_loc=E_loc, e_lo=e_lo, k=k, cf=cf, dtype="f16")
    desc = B.desc_from_shape(shape)
    R_max = B.moe_max_rows(desc)
    ws = torch.empty(max(B.moe_workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    x = (torch.arange(T * 64, device="cuda", dtype=torch.float32).reshape(T, 64) % 1000).half()
    d_idx = torch.tensor(idx, dtype=torch.int32, device="cuda")
    demand = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    slot_token = torch.full((max(R_max, 1),), 12345, dtype=torch.int32, device="cuda")
    token_slot = torch.empty((T, k), dtype=torch.int32, device="cuda")
    x_disp = torch.empty((max(R_max, 1), 64), dtype=torch.float16, device="cuda")
    B.moe_dispatch(desc, d_idx, x, demand, offsets, slot_token, token_slot, x_disp, ws)
    torch.cuda.synchronize()
    assert np.array_equal(G.host(demand), ref["demand"])
    assert np.array_equal(G.host(offsets), ref["offsets"])
    assert np.array_equal(G.host(token_slot), ref["token_slot"])
    st = G.host(slot_token)[:R_max]
    assert np.array_equal(st[: ref["R"]], ref["slot_token"])
    assert np.all(st[ref["R"]:] == -1)
    assert np.array_equal(G.host(x_disp)[: ref["R"]], G.host(x)[ref["slot_token"]])


@pytest.mark.parametrize("k", [1, 2])
def test_combine_exact_payload(k):
    """fp32 rows holding their own slot number and unit weights: each output row
    must be exactly the sum of its kept slots' numbers (0 when all dropped)."""
    T, E, H = 300, 8, 64
    rng = np.random.default_rng(5 + k)
    idx, _ = oracle.top_k(rng.standard_normal((T, E)), k)
    cf = 0.5
    C = oracle.capacity(T, E, k, cf)
    d = oracle.dispatch(idx, E, C)
    shape = W.LayerShape("comb", T=T, H=H, F=64, E=E, E_loc=E, k=k, cf=cf, dtype="f32")
    desc = B.desc_from_shape(shape)
    R_max = B.moe_max_rows(desc)
    y_disp = torch.arange(R_max, dtype=torch.float32, device="cuda")[:, None].repeat(1, H).contiguous()
    wts = np.ones((T, k), dtype=np.float32)
    if k == 2:
        wts[:, 1] = 1024.0
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    B.moe_combine(desc, y_disp, torch.tensor(d["token_slot"], dtype=torch.int32, device="cuda"),
                  torch.tensor(wts, device="cuda"), None, y)
    torch.cuda.synchronize()
    ts = d["token_slot"]
    expect = np.where(ts[:, 0] >= 0, ts[:, 0], 0).astype(np.float64)
    if k == 2:
        expect = expect + 1024.0 * np.where(ts[:, 1] >= 0, ts[:, 1], 0)
    assert (ts < 0).any()
    assert np.array_equal(G.host(y), np.repeat(expect[:, None], H, axis=1))


def test_exact_logit_ties_pick_lower_index():
    """Duplicated gate rows give bit-identical logits; the lower expert must win."""
    for T in (40, 512):        # one-wave-per-expert path and matrix-core path
        shape = W.LayerShape("ties", T=T, H=256, F=256, E=64, E_loc=64, k=2, cf=4.0, dtype="f16")
        x, w = G.device_case(shape, seed=3)
        gw = w["gate_w"]
        gw[5] = gw[1]
        gw[7] = gw[2]
        g = G.gpu_steps(shape, x, w)
        idx = g["idx"]
        for t in range(T):
            row = list(idx[t])
            for lo, hi in ((1, 5), (2, 7)):
                if hi in row:
                    assert lo in row and row.index(lo) < row.index(hi), (T, t, row)
        assert (np.isin(idx, [1, 2])).any()


def test_hot_expert_all_to_one():
    """Gate bias routes every token to expert 0: C rows kept, the rest dropped."""
    shape = W.LayerShape("hot", T=512, H=256, F=512, E=16, E_loc=16, k=1, cf=1.0, dtype="f16")
    x, w = G.device_case(shape, seed=4)
    b = torch.zeros(16, dtype=torch.float32, device="cuda")
    b[0] = 100.0
    w["gate_b"] = b
    g = G.gpu_steps(shape, x, w)
    C = oracle.capacity(512, 16, 1, 1.0)
    assert g["demand"][0] == 512 and g["R"] == C
    assert np.all(g["token_slot"][:C, 0] == np.arange(C)) and np.all(g["token_slot"][C:, 0] == -1)
    assert np.all(g["y"][C:] == 0)
    hx, hw = G.host(x), G.host_weights(w)
    ref = oracle.layer_forward(hx, hw, E=16, k=1, cf=1.0)
    G.assert_close(g["y"], ref["y"], "f16", "hot expert output")


def test_local_shares_sum_to_full_layer():
    full = R["share_reduced"].with_(E_loc=32, e_lo=0)
    x, wf = G.device_case(full, seed=0)
    yf = B.MoELayer(full, wf).forward(x).float()
    acc = torch.zeros_like(yf)
    for lo in range(0, 32, 8):
        sh = R["share_reduced"].with_(e_lo=lo)
        _, ws_ = G.device_case(sh, seed=0)
        acc += B.MoELayer(sh, ws_).forward(x).float()
    torch.cuda.synchronize()
    G.assert_close(G.host(acc), G.host(yf), "f16", "sum of 4 shares vs full layer")


@pytest.mark.parametrize("dtype,E,gate", [("f16", 16, "vector"), ("bf16", 16, "vector"), ("f16", 64, "matrix"),
                                          ("bf16", 64, "matrix")])
def test_folded_combine_without_kept_rows(dtype, E, gate):
    """A top-1 layer whose local experts receive no token (the gate bias sends
    every token to expert 0): neither grouped GEMM has a tile, and every row of
    y (filled with 7s before) is still zeroed, by the dispatch (vector-ALU gate)
    or by the matrix-core gate's work-groups, which is the oracle's combine for
    tokens without a kept local choice."""
    shape = W.LayerShape("nokept", T=300, H=256, F=512, E=E, E_loc=2, e_lo=8, k=1, cf=2.0, dtype=dtype)
    G.say(f"[no kept rows] {dtype} E={E}")
    plan = B.moe_layer_plan(B.desc_from_shape(shape))
    assert plan["expert_path"] == "grouped_gemm" and plan["combine_in_expert_kernel"], plan
    assert plan["gate_path"] == gate, plan
    x, w = G.device_case(shape, seed=5)
    w["gate_w"] = torch.zeros_like(w["gate_w"])
    gb = torch.zeros(shape.E, dtype=torch.float32, device="cuda")
    gb[0] = 4.0
    w["gate_b"] = gb
    hx, hw = G.host(x), G.host_weights(w)
    route = oracle.route(hx, hw["gate_w"], hw["gate_b"], shape.k, False)
    assert np.all(route["idx"] == 0)
    y = torch.full_like(x, 7.0)
    B.MoELayer(shape, w).forward(x, y)
    torch.cuda.synchronize()
    assert int((y != 0).sum()) == 0


def test_dispatch_zero_tokens():
    shape = W.LayerShape("empty", T=0, H=64, F=64, E=8, E_loc=8, k=1, cf=1.0, dtype="f16")
    desc = B.desc_from_shape(shape)
    demand = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    B.moe_dispatch(desc, None, None, demand, offsets, None, None, None, None)
    torch.cuda.synchronize()
    assert int(demand.abs().sum()) == 0 and int(offsets.abs().sum()) == 0
