"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import erf

import oracle.moe_oracle as M
from tests import oracle_pins as P

_orig = {n: getattr(M, n) for n in ("top_k", "dispatch", "gelu", "softmax", "capacity", "combine",
                                    "ffn", "combine_weights", "gate_logits", "layer_rows", "route")}


def _ties_to_higher(z, k):
    z = np.asarray(z, dtype=np.float64)
    T, E = z.shape
    order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -z), axis=-1)
    idx, margin = _orig["top_k"](z, k)
    return order[:, :k].astype(np.int64), margin


def _token_major(idx, E, C, e_lo=0, E_loc=None):
    # walk tokens first, then choices: a token's second choice outranks later tokens' first
    idx = np.asarray(idx)
    T, k = idx.shape
    perm = np.zeros_like(idx)
    d = _orig["dispatch"](idx, E, C, e_lo, E_loc)
    count = [0] * E
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j]); perm[t, j] = count[e]; count[e] += 1
    E_loc = E - e_lo if E_loc is None else E_loc
    off = d["offsets"]
    ts = np.full((T, k), -1, dtype=np.int64)
    st = np.full(d["R"], -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e_lo <= e < e_lo + E_loc and perm[t, j] < C:
                ts[t, j] = off[e - e_lo] + perm[t, j]; st[ts[t, j]] = t
    d = dict(d, pos=perm, token_slot=ts, slot_token=st)
    return d


def _keep_le(idx, E, C, e_lo=0, E_loc=None):
    return _orig["dispatch"](idx, E, C + 1, e_lo, E_loc)


def _tanh_gelu(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))


def _softmax_no_norm(z):
    z = np.asarray(z, dtype=np.float64)
    return np.exp(z - z.max(axis=1, keepdims=True))


def _capacity_floor(T, E, k, cf):
    return int(math.floor(Fraction(cf) * k * T / E))


def _combine_unweighted(y_disp, token_slot, w, T, H, dense=None):
    return _orig["combine"](y_disp, token_slot, np.ones_like(np.asarray(w, dtype=np.float64)), T, H, dense)


def _combine_no_dense(y_disp, token_slot, w, T, H, dense=None):
    return _orig["combine"](y_disp, token_slot, w, T, H, None)


def _ffn_no_b2(x_rows, w1, b1, w2, b2):
    return _orig["ffn"](x_rows, w1, b1, w2, np.zeros_like(np.asarray(b2, dtype=np.float64)))


def _ffn_gelu_erf_halved(x_rows, w1, b1, w2, b2):
    x = np.asarray(x_rows, dtype=np.float64)
    u = x @ np.asarray(w1, np.float64).T + np.asarray(b1, np.float64)
    h = u * 0.5 * (1 + erf(u))          # forgot the 1/sqrt(2)
    return h @ np.asarray(w2, np.float64).T + np.asarray(b2, np.float64)


def _gate_no_bias(x, gate_w, gate_b=None):
    return _orig["gate_logits"](x, gate_w, None)


def _rows_variant(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights=None, *,
                  expert_of=None, weight_of=None, dense_per_choice=False):
    """layer_rows with one step changed (the planted mistakes below)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    n, H = x_rows.shape
    y = np.zeros((n, H))
    if dense_weights is not None and not dense_per_choice:
        y += M.ffn(x_rows, *dense_weights)
    dense = M.ffn(x_rows, *dense_weights) if dense_weights is not None else None
    for i in range(n):
        for j in range(token_slot_rows.shape[1]):
            s = int(token_slot_rows[i, j])
            if s < 0:
                continue
            e = expert_of(s) if expert_of else int(slot_expert[s])
            wt = weight_of(i, j) if weight_of else float(w_rows[i, j])
            y[i] += wt * M.ffn(x_rows[i:i + 1], *expert_weights[e])[0]
            if dense_per_choice and dense is not None:
                y[i] += dense[i]
    return y


def _rows_neighbour_expert(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights=None):
    # the expert of the slot before (wrong at every segment start)
    return _rows_variant(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights,
                         expert_of=lambda s: int(slot_expert[max(s - 1, 0)]))


def _rows_unweighted(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights=None):
    return _rows_variant(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights,
                         weight_of=lambda i, j: 1.0)


def _rows_first_choice_weight(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights=None):
    # every choice weighted by the token's first-choice weight
    return _rows_variant(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights,
                         weight_of=lambda i, j: float(w_rows[i, 0]))


def _rows_dense_per_choice(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights=None):
    # the dense MLP added once per kept choice (pass-through rows lose it)
    return _rows_variant(x_rows, token_slot_rows, w_rows, slot_expert, expert_weights, dense_weights,
                         dense_per_choice=True)


def _route_override_ignored(x, gate_w, gate_b, k, renorm=False, override=None):
    return _orig["route"](x, gate_w, gate_b, k, renorm, None)


def _route_override_keeps_weights(x, gate_w, gate_b, k, renorm=False, override=None):
    # adopts the experts but keeps the weights of the plain top-k
    r = _orig["route"](x, gate_w, gate_b, k, renorm, override)
    plain = _orig["route"](x, gate_w, gate_b, k, renorm, None)
    return dict(r, w=plain["w"])


MUTATIONS = {
    "rows_neighbour_slot_expert": ("layer_rows", _rows_neighbour_expert),
    "rows_ignore_weight": ("layer_rows", _rows_unweighted),
    "rows_first_choice_weight": ("layer_rows", _rows_first_choice_weight),
    "rows_dense_per_choice": ("layer_rows", _rows_dense_per_choice),
    "route_override_ignored": ("route", _route_override_ignored),
    "route_override_stale_weights": ("route", _route_override_keeps_weights),
    "ties_to_higher_index": ("top_k", _ties_to_higher),
    "token_major_priority": ("dispatch", _token_major),
    "keep_pos_le_C": ("dispatch", _keep_le),
    "tanh_gelu": ("gelu", _tanh_gelu),
    "softmax_unnormalised": ("softmax", _softmax_no_norm),
    "capacity_floor": ("capacity", _capacity_floor),
    "combine_ignores_weight": ("combine", _combine_unweighted),
    "residual_mlp_dropped": ("combine", _combine_no_dense),
    "ffn_drops_b2": ("ffn", _ffn_no_b2),
    "gelu_erf_scale": ("ffn", _ffn_gelu_erf_halved),
    "gate_ignores_bias": ("gate_logits", _gate_no_bias),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(M, attr, fn)
    failures = 0
    for check in P.ALL_CHECKS:
        try:
            check(M)
        except (AssertionError, ValueError, IndexError, KeyError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {name}"
