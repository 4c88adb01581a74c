"""Pins for the fp64 oracle: closed forms, invariants and brute force.

Each check takes the oracle module as an argument so the mutation tests can
run the same checks against an oracle with a planted mistake and see them
fail. Independent arithmetic comes from textbook values (tests/golden),
brute-force loops written differently from the oracle, and torch's float64
CPU routines (F.linear / F.gelu), never from the oracle itself.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as Fn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def torch_ffn(x, w1, b1, w2, b2):
    """Textbook dense FFN in torch float64: linear -> exact GeLU -> linear."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    h = Fn.gelu(Fn.linear(t(x), t(w1), t(b1)), approximate="none")
    return Fn.linear(h, t(w2), t(b2)).numpy()


def tiny_layer(rng, T, H, F, E, E_loc=None, residual=False, dup_rows=()):
    E_loc = E if E_loc is None else E_loc
    w = dict(
        gate_w=rng.standard_normal((E, H)) / math.sqrt(H),
        gate_b=None,
        w1=rng.standard_normal((E_loc, F, H)) * 0.3,
        b1=rng.standard_normal((E_loc, F)) * 0.1,
        w2=rng.standard_normal((E_loc, H, F)) * 0.3,
        b2=rng.standard_normal((E_loc, H)) * 0.1,
    )
    for a, b in dup_rows:
        w["gate_w"][b] = w["gate_w"][a]
    if residual:
        w.update(mlp_w1=rng.standard_normal((F, H)) * 0.3, mlp_b1=rng.standard_normal(F) * 0.1,
                 mlp_w2=rng.standard_normal((H, F)) * 0.3, mlp_b2=rng.standard_normal(H) * 0.1)
    x = rng.standard_normal((T, H))
    return x, w


# --------------------------------------------------------------------------- softmax
def check_softmax(O):
    for E in (1, 2, 3, 8, 128):
        p = O.softmax(np.full((3, E), 0.7))
        assert np.allclose(p, 1.0 / E, rtol=0, atol=1e-15)
    # two experts with logit gap d: the logistic function
    for d in (-3.0, -0.25, 0.0, 1e-6, 2.0, 30.0):
        p = O.softmax(np.array([[d, 0.0]]))
        assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(-d))) < 1e-15
        assert abs(p[0, 1] - 1.0 / (1.0 + math.exp(d))) < 1e-15
    # E = 1 is exactly one; large logits do not overflow; sums are one
    assert O.softmax(np.array([[1e6]]))[0, 0] == 1.0
    z = np.random.default_rng(1).standard_normal((50, 17)) * 40
    p = O.softmax(z)
    assert np.all(np.abs(p.sum(1) - 1) <= 1e-12)
    # ratio property p_a / p_b = exp(z_a - z_b)
    r = p[:, 3] / p[:, 5]
    assert np.allclose(np.log(r), z[:, 3] - z[:, 5], rtol=0, atol=1e-9)


# --------------------------------------------------------------------------- gelu
def check_gelu(O):
    g = load_golden("normal_cdf.json")["values"]
    for u_s, phi in g.items():
        u = float(u_s)
        got = float(O.gelu(np.array([u]))[0])
        assert abs(got - u * phi) <= 1e-15 * max(1.0, abs(u)), (u, got, u * phi)
    u = np.linspace(-6, 6, 241)
    # gelu(-u) = gelu(u) - u  (from Phi(-u) = 1 - Phi(u)); large u -> u; large -u -> 0
    assert np.allclose(O.gelu(-u), O.gelu(u) - u, rtol=0, atol=1e-14)
    assert abs(O.gelu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.gelu(np.array([-40.0]))[0]) < 1e-12


# --------------------------------------------------------------------------- top-k
def brute_topk(z, k):
    """Repeated first-occurrence argmax with the winner removed."""
    z = np.array(z, dtype=np.float64)
    T, E = z.shape
    idx = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        row = list(z[t])
        taken = set()
        for j in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or row[e] > row[best]:
                    best = e
            idx[t, j] = best
            taken.add(best)
    return idx


def check_topk(O):
    rng = np.random.default_rng(7)
    for k in (1, 2):
        z = rng.integers(-3, 4, size=(200, 6)).astype(np.float64)   # many exact ties
        idx, margin = O.top_k(z, k)
        assert np.array_equal(idx, brute_topk(z, k))
        for t in range(200):
            srt = sorted(z[t], reverse=True)
            m = min(srt[i] - srt[i + 1] for i in range(k))
            assert margin[t] == m
    z = rng.standard_normal((10, 2))
    _, margin = O.top_k(z, 2)
    assert np.all(np.isinf(margin))
    # gate with duplicated expert rows: exact logit ties, the lower index must win
    x, w = tiny_layer(rng, T=64, H=8, F=4, E=5, dup_rows=[(1, 3), (0, 4)])
    z = O.gate_logits(x, w["gate_w"])
    assert np.array_equal(z[:, 3], z[:, 1]) and np.array_equal(z[:, 4], z[:, 0])
    idx, _ = O.top_k(z, 2)
    for t in range(64):
        row = list(idx[t])
        for lo, hi in ((1, 3), (0, 4)):
            if hi in row:
                assert lo in row and row.index(lo) < row.index(hi)


# --------------------------------------------------------------------------- gate logits
def check_gate_logits(O):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7))
    wg = rng.standard_normal((4, 7))
    b = rng.standard_normal(4)
    z = O.gate_logits(x, wg, b)
    for t in range(5):
        for e in range(4):
            s = math.fsum(float(x[t, h]) * float(wg[e, h]) for h in range(7)) + float(b[e])
            assert abs(z[t, e] - s) < 1e-13


# --------------------------------------------------------------------------- capacity
def check_capacity(O):
    for c in load_golden("capacity.json")["cases"]:
        assert O.capacity(c["T"], c["E"], c["k"], c["cf"]) == c["C"], c
    for T, E, k, cf in itertools.product((1, 7, 64, 1000), (1, 2, 8), (1, 2), (0.5, 1.0, 1.25, 2.0, 8.0)):
        if k > E:
            continue
        C = O.capacity(T, E, k, cf)
        assert (C - 1) * E < k * T * cf <= C * E + 1e-9
        if cf * k >= E:
            assert C >= T


# --------------------------------------------------------------------------- dispatch
def brute_dispatch(idx, E, C, e_lo, E_loc):
    """O(n^2) positions: count earlier assignments (rank-major) with the same expert."""
    T, k = idx.shape
    order = [(j, t) for j in range(k) for t in range(T)]
    pos = {}
    for a, (j, t) in enumerate(order):
        e = idx[t, j]
        pos[(t, j)] = sum(1 for (j2, t2) in order[:a] if idx[t2, j2] == e)
    kept_e = {}
    for e in range(e_lo, e_lo + E_loc):
        kept_e[e] = sum(1 for (t, j) in pos if idx[t, j] == e and pos[(t, j)] < C)
    seg_start, acc = {}, 0
    for e in range(e_lo, e_lo + E_loc):
        seg_start[e] = acc
        acc += kept_e[e]
    token_slot = -np.ones((T, k), dtype=np.int64)
    for (t, j), p in pos.items():
        e = idx[t, j]
        if e_lo <= e < e_lo + E_loc and p < C:
            token_slot[t, j] = seg_start[e] + p
    demand = np.array([int(np.sum(idx == e)) for e in range(E)])
    return pos, demand, token_slot, acc


def check_dispatch(O):
    rng = np.random.default_rng(11)
    for trial in range(40):
        E = int(rng.integers(1, 6))
        k = int(rng.integers(1, min(2, E) + 1))
        T = int(rng.integers(0, 14))
        z = rng.standard_normal((T, E))
        idx, _ = O.top_k(z, k) if T else (np.zeros((0, k), dtype=np.int64), None)
        C = int(rng.integers(0, 5))
        e_lo = int(rng.integers(0, E))
        E_loc = int(rng.integers(1, E - e_lo + 1))
        d = O.dispatch(idx, E, C, e_lo, E_loc)
        pos, demand, token_slot, R = brute_dispatch(idx, E, C, e_lo, E_loc)
        assert np.array_equal(d["demand"], demand)
        assert np.array_equal(d["token_slot"], token_slot)
        assert d["R"] == R
        for (t, j), p in pos.items():
            assert d["pos"][t, j] == p
        # invariants
        off = d["offsets"]
        assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == R
        assert np.all(d["kept"] <= C)
        assert sum(d["kept"]) == sum(min(demand[e], C) for e in range(e_lo, e_lo + E_loc))
        seen = set()
        for t in range(T):
            for j in range(k):
                s = d["token_slot"][t, j]
                e = idx[t, j]
                if s >= 0:
                    assert s not in seen
                    seen.add(s)
                    assert d["slot_token"][s] == t
                    assert off[e - e_lo] <= s < off[e - e_lo + 1]
                    assert d["pos"][t, j] < C
                else:
                    assert d["pos"][t, j] >= C or not (e_lo <= e < e_lo + E_loc)
        assert len(seen) == R


def check_rank_major_priority(O):
    # token 1's first choice (expert 0) must beat token 0's second choice (expert 0)
    idx = np.array([[1, 0], [0, 1]])
    d = O.dispatch(idx, E=2, C=1)
    assert d["token_slot"][1, 0] == 0          # expert 0 slot 0 goes to token 1, first choice
    assert d["token_slot"][0, 1] == -1         # token 0's second choice is dropped
    assert d["token_slot"][0, 0] == 1          # expert 1's slot goes to token 0 first choice


# --------------------------------------------------------------------------- FFN / layer
def check_single_expert_is_dense_ffn(O):
    rng = np.random.default_rng(5)
    x, w = tiny_layer(rng, T=9, H=6, F=10, E=1)
    out = O.layer_forward(x, w, E=1, k=1, cf=1.0)
    ref = torch_ffn(x, w["w1"][0], w["b1"][0], w["w2"][0], w["b2"][0])
    assert np.allclose(out["y"], ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(out["p"], 1.0)


def brute_dense_mixture(O_route, x, w, E, k, C, e_lo, E_loc, renorm=False):
    """Every expert on every token, masked by the brute-force keep decision."""
    T = x.shape[0]
    z = x @ w["gate_w"].T + (0 if w.get("gate_b") is None else w["gate_b"])
    ez = np.exp(z - z.max(1, keepdims=True))
    p = ez / ez.sum(1, keepdims=True)
    idx = brute_topk(z, k)
    pos, _, token_slot, _ = brute_dispatch(idx, E, C, e_lo, E_loc)
    y = np.zeros_like(x, dtype=np.float64)
    for i in range(E_loc):
        e = e_lo + i
        ye = torch_ffn(x, w["w1"][i], w["b1"][i], w["w2"][i], w["b2"][i])
        for t in range(T):
            sel = [j for j in range(k) if idx[t, j] == e and token_slot[t, j] >= 0]
            if sel:
                wt = p[t, e]
                if renorm:
                    wt = wt / sum(p[t, idx[t, jj]] for jj in range(k))
                y[t] += wt * ye[t]
    return y


def check_layer_vs_dense_mixture(O):
    rng = np.random.default_rng(13)
    for (T, H, F, E, k, cf, renorm) in [(24, 6, 8, 4, 1, 1.0, False), (30, 5, 7, 5, 2, 0.75, False),
                                        (17, 4, 6, 3, 2, 1.0, True), (12, 4, 4, 6, 2, 3.0, False)]:
        x, w = tiny_layer(rng, T, H, F, E)
        C = O.capacity(T, E, k, cf)
        out = O.layer_forward(x, w, E=E, k=k, cf=cf, renorm=renorm)
        ref = brute_dense_mixture(None, x, w, E, k, C, 0, E, renorm)
        assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def check_residual(O):
    rng = np.random.default_rng(17)
    x, w = tiny_layer(rng, T=20, H=5, F=8, E=4, residual=True)
    std = O.layer_forward(x, w, E=4, k=1, cf=1.0)
    res = O.layer_forward(x, w, E=4, k=1, cf=1.0, residual=True)
    mlp = torch_ffn(x, w["mlp_w1"], w["mlp_b1"], w["mlp_w2"], w["mlp_b2"])
    assert np.allclose(res["y"], std["y"] + mlp, rtol=1e-12, atol=1e-12)
    # a share holding only expert 0: every other token passes through the MLP alone
    share = O.layer_forward(x, dict(w, w1=w["w1"][:1], b1=w["b1"][:1], w2=w["w2"][:1], b2=w["b2"][:1]),
                            E=4, k=1, cf=1.0, residual=True, E_loc=1, e_lo=0)
    passthru = share["token_slot"][:, 0] < 0
    assert passthru.sum() > 0
    assert np.allclose(share["y"][passthru], mlp[passthru], rtol=1e-12, atol=1e-12)
    # one expert: y = MLP(x) + FFN_0(x)
    x1, w1 = tiny_layer(rng, T=6, H=4, F=5, E=1, residual=True)
    one = O.layer_forward(x1, w1, E=1, k=1, cf=1.0, residual=True)
    ref = torch_ffn(x1, w1["mlp_w1"], w1["mlp_b1"], w1["mlp_w2"], w1["mlp_b2"]) + \
        torch_ffn(x1, w1["w1"][0], w1["b1"][0], w1["w2"][0], w1["b2"][0])
    assert np.allclose(one["y"], ref, rtol=1e-12, atol=1e-12)


def check_local_shares_sum(O):
    rng = np.random.default_rng(19)
    T, H, F, E, k, cf = 40, 5, 6, 8, 2, 1.0
    x, w = tiny_layer(rng, T, H, F, E)
    full = O.layer_forward(x, w, E=E, k=k, cf=cf)
    acc = np.zeros_like(full["y"])
    for lo in range(0, E, 2):
        ws = dict(w, w1=w["w1"][lo:lo + 2], b1=w["b1"][lo:lo + 2], w2=w["w2"][lo:lo + 2],
                  b2=w["b2"][lo:lo + 2])
        share = O.layer_forward(x, ws, E=E, k=k, cf=cf, e_lo=lo, E_loc=2)
        assert np.array_equal(share["demand"], full["demand"])
        acc += share["y"]
    assert np.allclose(acc, full["y"], rtol=1e-12, atol=1e-12)


def check_linearity_and_permutation(O):
    rng = np.random.default_rng(23)
    T, H, F, E = 16, 5, 7, 4
    x, w = tiny_layer(rng, T, H, F, E)
    base = O.layer_forward(x, w, E=E, k=2, cf=0.5)
    ws = dict(w, w2=w["w2"] * 3.0, b2=w["b2"] * 3.0)
    scaled = O.layer_forward(x, ws, E=E, k=2, cf=0.5)
    assert np.allclose(scaled["y"], 3.0 * base["y"], rtol=1e-12, atol=1e-12)
    # without drops the layer is row-wise: permuting tokens permutes outputs
    nodrop = O.layer_forward(x, w, E=E, k=2, cf=float(E))
    perm = rng.permutation(T)
    pd = O.layer_forward(x[perm], w, E=E, k=2, cf=float(E))
    assert np.allclose(pd["y"], nodrop["y"][perm], rtol=1e-12, atol=1e-12)
    # relabelling experts (gate rows and expert weights together) changes nothing
    q = rng.permutation(E)
    wq = dict(gate_w=w["gate_w"][q], gate_b=None, w1=w["w1"][q], b1=w["b1"][q], w2=w["w2"][q],
              b2=w["b2"][q])
    rq = O.layer_forward(x, wq, E=E, k=2, cf=float(E))
    assert np.allclose(rq["y"], nodrop["y"], rtol=1e-12, atol=1e-12)


class OnlyExperts(dict):
    """Expert weights for the experts a sample needs; any other lookup fails (the
    full-size tests hand layer_rows a mapping that loads one expert at a time)."""

    def __getitem__(self, e):
        if e not in self.keys():
            raise KeyError(f"expert {e} was not expected to be needed")
        return dict.__getitem__(self, e)


def check_layer_rows(O):
    """layer_rows (output rows for a sample of tokens, given their routing) equals
    the brute-force dense mixture (+ the dense MLP in residual mode) on those rows:
    top-1 and top-2, drops, residual layers with pass-through rows, local shares,
    rows sampled out of order and with repeats."""
    rng = np.random.default_rng(29)
    #        T   H  F  E  k  cf    e_lo E_loc residual
    cases = [(24, 5, 7, 4, 1, 1.0, 0, 4, False),
             (30, 5, 6, 5, 2, 0.75, 0, 5, False),
             (28, 4, 6, 6, 2, 1.0, 2, 3, False),
             (20, 5, 8, 4, 1, 0.5, 0, 4, True),
             (26, 4, 5, 6, 1, 1.0, 1, 2, True)]
    for T, H, F, E, k, cf, e_lo, E_loc, residual in cases:
        x, w = tiny_layer(rng, T, H, F, E, E_loc, residual)
        C = O.capacity(T, E, k, cf)
        r = O.route(x, w["gate_w"], w["gate_b"], k)
        d = O.dispatch(r["idx"], E, C, e_lo, E_loc)
        slot_expert = np.repeat(np.arange(E_loc), np.diff(d["offsets"]))
        rows = np.concatenate([rng.permutation(T)[: T - 3], [0, 0]])
        used = {int(slot_expert[s]) for s in d["token_slot"][rows].ravel() if s >= 0}
        ew = OnlyExperts({e: (w["w1"][e], w["b1"][e], w["w2"][e], w["b2"][e]) for e in used})
        dense = (w["mlp_w1"], w["mlp_b1"], w["mlp_w2"], w["mlp_b2"]) if residual else None
        got = O.layer_rows(x[rows], d["token_slot"][rows], r["w"][rows], slot_expert, ew, dense)
        ref = brute_dense_mixture(None, x, w, E, k, C, e_lo, E_loc)
        if residual:
            ref = ref + torch_ffn(x, *dense)
        assert np.allclose(got, ref[rows], rtol=1e-12, atol=1e-12)
        # the cases must reach what they are there for
        kept = d["token_slot"] >= 0
        assert kept.any()
        if cf < 1.0 or E_loc < E - e_lo or e_lo > 0:
            assert (~kept).any()


def check_route_override(O):
    """route with an override (the tests adopt the GPU's legal choice for near-tie
    tokens) takes the given experts for those tokens, the softmax probabilities at
    them as weights, and leaves every other token as the plain top-k."""
    rng = np.random.default_rng(31)
    x, w = tiny_layer(rng, T=12, H=6, F=4, E=5)
    plain = O.route(x, w["gate_w"], None, 2)
    over = {3: np.array([4, 0]), 7: np.array([1, 2])}
    r = O.route(x, w["gate_w"], None, 2, override=over)
    z = x @ w["gate_w"].T
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    for t in range(12):
        want = over[t] if t in over else brute_topk(z[t:t + 1], 2)[0]
        assert np.array_equal(r["idx"][t], want)
        assert np.allclose(r["w"][t], p[t, want], rtol=1e-13, atol=1e-15)
        if t not in over:
            assert np.array_equal(r["idx"][t], plain["idx"][t])


ALL_CHECKS = [check_softmax, check_gelu, check_topk, check_gate_logits, check_capacity,
              check_dispatch, check_rank_major_priority, check_single_expert_is_dense_ffn,
              check_layer_vs_dense_mixture, check_residual, check_local_shares_sum,
              check_linearity_and_permutation, check_layer_rows, check_route_override]
