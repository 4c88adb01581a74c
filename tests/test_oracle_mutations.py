"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import erf

import oracle.moe_oracle as M
from tests import oracle_pins as P

_orig = {n: getattr(M, n) for n in ("top_k", "dispatch", "gelu", "softmax", "capacity", "combine",
                                    "ffn", "combine_weights", "gate_logits")}


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


MUTATIONS = {
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
