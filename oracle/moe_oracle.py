"""fp64 CPU oracle for the forward pass of one DeepSpeed-MoE-style MoE FFN layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP
library and imports nothing from it.

Everything is plain NumPy in float64. Inputs may be float16 / float32 /
float64 arrays; they are widened exactly, nothing is ever rounded back to a
narrow type. The steps follow the pages in their order:

  1. gate logits z = x Wg^T (+ b)          "[Review] DeepSpeed-MoE", "What is MoE?"
                                           (Switch-Transformer layer: a gating
                                           function routes each token to expert FFNs)
  2. p = softmax over all E experts        "Fast MoE Inference via Predictive
                                           Prefetching and Expert Replication",
                                           problem statement (softmax-based routing)
  3. top-k experts by logit, ties to the   same review, "MoE based NLG Model
     lower expert index                    Architecture" (top-1: as many active
                                           parameters per token as the dense model)
                                           and "Phenomenon2" (Top2-MoE)
  4. capacity C = ceil(k T cf / E)         (the pages print no formula: plainest
                                           reading, global E, no minimum floor)
  5. dispatch in rank-major priority,      (the pages are silent on priority: every
     drop assignments past C               first choice outranks every second
                                           choice, lower token first; a dropped
                                           assignment contributes exactly zero)
  6. expert FFN  GeLU(x W1^T + b1) W2^T + b2 with exact (erf) GeLU
  7. combine  y[t] = sum_j w[t,j] FFN_{e_j}(x_t) over kept local assignments
  8. residual mode (PR-MoE)  y += MLP(x)   same review, "Phenomenon2"
                                           (Residual-MoE: fixed MLP plus one routed
                                           expert, summed) and "PR-MoE: Pyramid-
                                           Residual-MoE"

Pins: every function here is checked against closed forms, invariants and
brute force in tests/test_oracle_pins.py. Beyond those checks, the *values*
of the layer output are "parity unpinned" by the pages (they print no worked
example); the pins are what ties the oracle to the method.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Mapping, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

_SQRT1_2 = 1.0 / math.sqrt(2.0)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- step 1-3: gate
def gate_logits(x, gate_w, gate_b=None) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * Wg[e, h] (+ b[e]).  Wg in nn.Linear layout [E, H]."""
    z = _f64(x) @ _f64(gate_w).T
    if gate_b is not None:
        z = z + _f64(gate_b)[None, :]
    return z


def softmax(z) -> np.ndarray:
    """Softmax over the expert axis (max-subtracted; mathematically exact form)."""
    z = _f64(z)
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def top_k(z, k: int):
    """Experts ordered by logit descending, ties to the lower expert index.

    Returns (idx [T, k] int64, margin [T] float64) where margin[t] is the
    smallest gap between consecutive logits among the first k+1 of the order
    (+inf when k == E): a token with a small margin may legally route either way.
    """
    z = _f64(z)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -z), axis=-1)
    idx = order[:, :k].astype(np.int64)
    if k == E:
        margin = np.full(T, np.inf)
    else:
        zs = np.take_along_axis(z, order[:, : k + 1], axis=1)
        margin = np.min(zs[:, :-1] - zs[:, 1:], axis=1)
    return idx, margin


def combine_weights(p, idx, renorm: bool = False) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]]; optionally divided by the sum over the selected experts."""
    w = np.take_along_axis(_f64(p), np.asarray(idx), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


# ---------------------------------------------------------------- step 4: capacity
def capacity(T: int, E: int, k: int, cf: float) -> int:
    """C = ceil(k * T * cf / E), computed exactly from the binary value of cf."""
    q = Fraction(cf) * k * T / E
    return int(math.ceil(q))


def max_rows(T: int, E_loc: int, k: int, C: int) -> int:
    """Upper bound on dispatched rows held by one GPU: min(E_loc * C, k * T)."""
    return min(E_loc * C, k * T)


# ---------------------------------------------------------------- step 5: dispatch
def dispatch(idx, E: int, C: int, e_lo: int = 0, E_loc: Optional[int] = None) -> dict:
    """Walk the assignments in rank-major order (every token's j-th choice before
    any token's (j+1)-th; tokens in index order within a rank), keep a running
    count per expert, and keep an assignment while its position is below C.

    Demand counts every assignment; only experts in [e_lo, e_lo + E_loc) get
    slots. Slots are numbered expert by expert (local order), then by position.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if E_loc is None:
        E_loc = E - e_lo
    count = [0] * E
    pos = np.zeros((T, k), dtype=np.int64)
    for j in range(k):
        for t in range(T):
            e = int(idx[t, j])
            pos[t, j] = count[e]
            count[e] += 1
    demand = np.array(count, dtype=np.int64)
    kept = np.array([min(demand[e_lo + i], C) for i in range(E_loc)], dtype=np.int64)
    offsets = np.zeros(E_loc + 1, dtype=np.int64)
    for i in range(E_loc):
        offsets[i + 1] = offsets[i] + kept[i]
    R = int(offsets[E_loc])
    token_slot = np.full((T, k), -1, dtype=np.int64)
    slot_token = np.full(R, -1, dtype=np.int64)
    slot_choice = np.full(R, -1, dtype=np.int64)
    for j in range(k):
        for t in range(T):
            e = int(idx[t, j])
            if e_lo <= e < e_lo + E_loc and pos[t, j] < C:
                s = int(offsets[e - e_lo] + pos[t, j])
                token_slot[t, j] = s
                slot_token[s] = t
                slot_choice[s] = j
    return dict(pos=pos, demand=demand, kept=kept, offsets=offsets, token_slot=token_slot,
                slot_token=slot_token, slot_choice=slot_choice, R=R)


# ---------------------------------------------------------------- step 6: expert FFN
def gelu(u) -> np.ndarray:
    """Exact GeLU: u * Phi(u) with Phi the standard normal CDF, via erf."""
    u = _f64(u)
    return u * 0.5 * (1.0 + _erf(u * _SQRT1_2))


def ffn(x_rows, w1, b1, w2, b2) -> np.ndarray:
    """GeLU(x W1^T + b1) W2^T + b2 for rows x [M, H]; W1 [F, H], W2 [H, F]."""
    h = gelu(_f64(x_rows) @ _f64(w1).T + _f64(b1)[None, :])
    return h @ _f64(w2).T + _f64(b2)[None, :]


def expert_outputs(x, dispatch_info, w1, b1, w2, b2) -> np.ndarray:
    """y_disp[s] = FFN_e(x[slot_token[s]]) for every dispatched slot s (local expert order)."""
    x = _f64(x)
    offsets = dispatch_info["offsets"]
    slot_token = dispatch_info["slot_token"]
    H = x.shape[1]
    y_disp = np.zeros((dispatch_info["R"], H))
    for i in range(len(offsets) - 1):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if b > a:
            y_disp[a:b] = ffn(x[slot_token[a:b]], w1[i], b1[i], w2[i], b2[i])
    return y_disp


# ---------------------------------------------------------------- step 7-8: combine
def combine(y_disp, token_slot, w, T: int, H: int, dense=None) -> np.ndarray:
    """y[t] = sum over kept local choices j of w[t, j] * y_disp[token_slot[t, j]]
    (+ dense[t] in residual mode). Rows with nothing kept get 0 (or dense[t])."""
    y = np.zeros((T, H)) if dense is None else _f64(dense).copy()
    token_slot = np.asarray(token_slot)
    w = _f64(w)
    for t in range(T):
        for j in range(token_slot.shape[1]):
            s = int(token_slot[t, j])
            if s >= 0:
                y[t] += w[t, j] * y_disp[s]
    return y


# ---------------------------------------------------------------- whole layer
def route(x, gate_w, gate_b, k: int, renorm: bool = False, override: Optional[dict] = None):
    """Gate + softmax + top-k + weights. `override` maps token -> expert list and
    replaces the top-k choice of that token (used only for near-tie adoption)."""
    z = gate_logits(x, gate_w, gate_b)
    p = softmax(z)
    idx, margin = top_k(z, k)
    if override:
        idx = idx.copy()
        for t, es in override.items():
            idx[t, :] = es
    w = combine_weights(p, idx, renorm)
    return dict(z=z, p=p, idx=idx, margin=margin, w=w)


def layer_forward(x, weights: Mapping, *, E: int, k: int, cf: float, e_lo: int = 0,
                  E_loc: Optional[int] = None, residual: bool = False, renorm: bool = False,
                  override: Optional[dict] = None) -> dict:
    """Full layer on host arrays. weights: gate_w [E,H], gate_b [E] or None,
    w1 [E_loc,F,H], b1 [E_loc,F], w2 [E_loc,H,F], b2 [E_loc,H], and in residual
    mode mlp_w1 [F,H], mlp_b1 [F], mlp_w2 [H,F], mlp_b2 [H]."""
    x = _f64(x)
    T, H = x.shape
    if E_loc is None:
        E_loc = E - e_lo
    if residual and k != 1:
        raise ValueError("residual mode routes exactly one expert per token")
    r = route(x, weights["gate_w"], weights.get("gate_b"), k, renorm, override)
    C = capacity(T, E, k, cf)
    d = dispatch(r["idx"], E, C, e_lo, E_loc)
    y_disp = expert_outputs(x, d, weights["w1"], weights["b1"], weights["w2"], weights["b2"])
    dense = None
    if residual:
        dense = ffn(x, weights["mlp_w1"], weights["mlp_b1"], weights["mlp_w2"], weights["mlp_b2"])
    y = combine(y_disp, d["token_slot"], r["w"], T, H, dense)
    out = dict(r)
    out.update(d)
    out.update(C=C, y_disp=y_disp, dense=dense, y=y)
    return out


def layer_rows(x_rows, token_slot_rows, w_rows, slot_expert: Sequence[int] | np.ndarray,
               expert_weights: Mapping[int, tuple], dense_weights: Optional[tuple] = None) -> np.ndarray:
    """Output rows for a sample of tokens, given their routing (step 7 on a subset).

    x_rows [n, H]; token_slot_rows [n, k] (slot or -1); w_rows [n, k];
    slot_expert maps a slot to its local expert; expert_weights[e] =
    (w1, b1, w2, b2) for every local expert the sampled kept slots use, looked
    up once per expert in increasing order (so a mapping may load them one at a
    time). Each expert's FFN runs once on the stack of sampled rows routed to it.
    In residual mode dense_weights = (w1, b1, w2, b2) of the MLP, added once to
    every row. Pinned against the brute-force dense mixture (every expert on
    every token, masked by a brute-force dispatch) in the oracle's pin checks.
    """
    x_rows = _f64(x_rows)
    n, H = x_rows.shape
    token_slot_rows = np.asarray(token_slot_rows)
    y = np.zeros((n, H))
    if dense_weights is not None:
        y += ffn(x_rows, *dense_weights)
    uses = {}
    for i in range(n):
        for j in range(token_slot_rows.shape[1]):
            s = int(token_slot_rows[i, j])
            if s >= 0:
                uses.setdefault(int(slot_expert[s]), []).append((i, j))
    for e, ij in sorted(uses.items()):
        rows = [i for i, _ in ij]
        ye = ffn(x_rows[rows], *expert_weights[e])
        for r, (i, j) in enumerate(ij):
            y[i] += float(w_rows[i, j]) * ye[r]
    return y
