"""ctypes binding of libmoe_mi355x (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch
tensors into device pointers and the current torch stream into a hipStream_t,
and raises MoeError for any status other than MOE_OK. It never computes a step
itself and has no fallback: without the built library every call fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_F16, MOE_DTYPE_BF16 = 0, 1, 2
MOE_MLP_STANDARD, MOE_MLP_RESIDUAL = 0, 1
MOE_FLAG_RENORM_TOPK = 1
MOE_FLAG_DECODE_ONE_LAUNCH = 2

EXPORTED = ["moe_capacity", "moe_max_rows", "moe_workspace_size", "moe_layer_plan", "moe_gate", "moe_dispatch",
            "moe_expert_ffn", "moe_dense_ffn", "moe_combine", "moe_layer_forward",
            "moe_layer_forward_ex", "moe_layer_forward_noalloc", "moe_status_str", "moe_last_error",
            "moe_expert_store_create", "moe_expert_store_destroy", "moe_expert_store_set_expert",
            "moe_expert_store_weights", "moe_expert_store_update", "moe_expert_store_update_async",
            "moe_expert_store_commit", "moe_expert_store_residency"]

_DTYPE_CODE = {torch.float32: MOE_DTYPE_F32, torch.float16: MOE_DTYPE_F16, torch.bfloat16: MOE_DTYPE_BF16}
_DTYPE_NAME = {"f32": MOE_DTYPE_F32, "f16": MOE_DTYPE_F16, "bf16": MOE_DTYPE_BF16}


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_name(status)}: {detail}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("first_local_expert", ctypes.c_int32),
                ("num_local_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("capacity_factor", ctypes.c_double), ("mlp_type", ctypes.c_int),
                ("dtype", ctypes.c_int), ("flags", ctypes.c_uint32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_w", "gate_b", "w1", "b1", "w2", "b2", "mlp_w1", "mlp_b1", "mlp_w2", "mlp_b2",
                 "w1_experts", "b1_experts", "w2_experts", "b2_experts")]


class LayerPlan(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int64), ("max_rows", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
                ("gate_path", ctypes.c_int), ("expert_path", ctypes.c_int),
                ("dispatch_in_expert_kernel", ctypes.c_int32), ("combine_in_expert_kernel", ctypes.c_int32),
                ("dense_in_expert_kernels", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("tile_cols_w1", ctypes.c_int32), ("tile_cols_w2", ctypes.c_int32),
                ("experts_one_launch", ctypes.c_int32)]


EXPERT_PATHS = {0: "grouped_gemm", 1: "stream"}


class PhaseEvents(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_begin", "gate_end", "dispatch_begin", "dispatch_end", "ffn_begin", "ffn_split",
                 "ffn_end", "combine_begin", "combine_end", "up_start", "up_stop", "down_start", "down_stop")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python mixture_experts_transformer_moe_amd/csrc/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        st = ctypes.c_int
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        L.moe_max_rows.restype = ctypes.c_int64
        L.moe_max_rows.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_workspace_size.restype = st
        L.moe_workspace_size.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(ctypes.c_size_t)]
        D = ctypes.POINTER(LayerDesc)
        W = ctypes.POINTER(LayerWeights)
        sz = ctypes.c_size_t
        L.moe_layer_plan.restype = st
        L.moe_layer_plan.argtypes = [D, ctypes.POINTER(LayerPlan)]
        L.moe_gate.restype = st
        L.moe_gate.argtypes = [D, P, P, P, P, P, P, P, sz, P]
        L.moe_dispatch.restype = st
        L.moe_dispatch.argtypes = [D, P, P, P, P, P, P, P, P, sz, P]
        L.moe_expert_ffn.restype = st
        L.moe_expert_ffn.argtypes = [D, P, P, W, P, P, sz, P]
        L.moe_dense_ffn.restype = st
        L.moe_dense_ffn.argtypes = [D, P, W, P, P, sz, P]
        L.moe_combine.restype = st
        L.moe_combine.argtypes = [D, P, P, P, P, P, P]
        L.moe_layer_forward.restype = st
        L.moe_layer_forward.argtypes = [D, W, P, P, P, sz, P]
        L.moe_layer_forward_noalloc.restype = st
        L.moe_layer_forward_noalloc.argtypes = [D, W, P, P, P]
        L.moe_layer_forward_ex.restype = st
        L.moe_layer_forward_ex.argtypes = [D, W, P, P, P, sz, P, ctypes.POINTER(PhaseEvents)]
        L.moe_expert_store_create.restype = st
        L.moe_expert_store_create.argtypes = [D, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
        L.moe_expert_store_destroy.restype = st
        L.moe_expert_store_destroy.argtypes = [P]
        L.moe_expert_store_set_expert.restype = st
        L.moe_expert_store_set_expert.argtypes = [P, ctypes.c_int32, P, P, P, P]
        L.moe_expert_store_weights.restype = st
        L.moe_expert_store_weights.argtypes = [P, W]
        L.moe_expert_store_update.restype = st
        L.moe_expert_store_update.argtypes = [P, P, P, ctypes.POINTER(ctypes.c_int32)]
        L.moe_expert_store_update_async.restype = st
        L.moe_expert_store_update_async.argtypes = [P, P, P, P, ctypes.POINTER(ctypes.c_int32)]
        L.moe_expert_store_commit.restype = st
        L.moe_expert_store_commit.argtypes = [P, P]
        L.moe_expert_store_residency.restype = st
        L.moe_expert_store_residency.argtypes = [P, P]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [st]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        _lib = L
    return _lib


def status_name(st: int) -> str:
    try:
        return lib().moe_status_str(st).decode()
    except Exception:
        return f"status {st}"


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def make_desc(T, H, F, E, k, cf, dtype, *, e_lo=0, E_loc=None, residual=False, renorm=False,
              one_launch=False) -> LayerDesc:
    if isinstance(dtype, torch.dtype):
        code = _DTYPE_CODE[dtype]
    elif isinstance(dtype, str):
        code = _DTYPE_NAME[dtype]
    else:
        code = int(dtype)
    return LayerDesc(num_tokens=T, hidden=H, ffn=F, num_experts=E, first_local_expert=e_lo,
                     num_local_experts=(E - e_lo) if E_loc is None else E_loc, top_k=k,
                     capacity_factor=float(cf), mlp_type=MOE_MLP_RESIDUAL if residual else MOE_MLP_STANDARD,
                     dtype=code, flags=(MOE_FLAG_RENORM_TOPK if renorm else 0) |
                     (MOE_FLAG_DECODE_ONE_LAUNCH if one_launch else 0))


def desc_from_shape(shape, T: Optional[int] = None) -> LayerDesc:
    """Descriptor for a workloads.LayerShape (optionally with another token count)."""
    return make_desc(shape.T if T is None else T, shape.H, shape.F, shape.E, shape.k, shape.cf, shape.dtype,
                     e_lo=shape.e_lo, E_loc=shape.E_loc, residual=shape.residual, renorm=shape.renorm,
                     one_launch=shape.one_launch)


def make_weights(w: dict) -> LayerWeights:
    return LayerWeights(**{n: (_ptr(w[n]) if w.get(n) is not None else None) for n, _ in LayerWeights._fields_})


# ---------------------------------------------------------------- the C entry points
def moe_capacity(T: int, E: int, k: int, cf: float) -> int:
    return lib().moe_capacity(T, E, k, cf)


def moe_max_rows(desc: LayerDesc) -> int:
    r = lib().moe_max_rows(ctypes.byref(desc))
    if r < 0:
        _check(MOE_ERR_INVALID_ARGUMENT)
    return r


def moe_workspace_size(desc: LayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def moe_layer_plan(desc: LayerDesc) -> dict:
    pl = LayerPlan()
    _check(lib().moe_layer_plan(ctypes.byref(desc), ctypes.byref(pl)))
    return dict(capacity=pl.capacity, max_rows=pl.max_rows, workspace_bytes=pl.workspace_bytes,
                gate_path="matrix" if pl.gate_path else "vector", expert_path=EXPERT_PATHS[pl.expert_path],
                dispatch_in_expert_kernel=bool(pl.dispatch_in_expert_kernel),
                combine_in_expert_kernel=bool(pl.combine_in_expert_kernel),
                dense_in_expert_kernels=bool(pl.dense_in_expert_kernels), launches=pl.launches,
                experts_one_launch=bool(pl.experts_one_launch),
                tile=(pl.tile_rows, pl.tile_cols_w1, pl.tile_cols_w2))


def _ws(ws: Optional[torch.Tensor]):
    return (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())


def moe_gate(desc, x, gate_w, gate_b, topk_idx, topk_w, probs=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_gate(ctypes.byref(desc), _ptr(x), _ptr(gate_w), _ptr(gate_b), _ptr(topk_idx), _ptr(topk_w),
                          _ptr(probs), p, n, _stream(stream)))


def moe_dispatch(desc, topk_idx, x, expert_demand, expert_offsets, slot_token, token_slot, x_disp=None, ws=None,
                 stream=None):
    p, n = _ws(ws)
    _check(lib().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(x), _ptr(expert_demand),
                              _ptr(expert_offsets), _ptr(slot_token), _ptr(token_slot), _ptr(x_disp), p, n,
                              _stream(stream)))


def moe_expert_ffn(desc, x_disp, expert_offsets, weights: LayerWeights, y_disp, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_expert_ffn(ctypes.byref(desc), _ptr(x_disp), _ptr(expert_offsets), ctypes.byref(weights),
                                _ptr(y_disp), p, n, _stream(stream)))


def moe_dense_ffn(desc, x, weights: LayerWeights, out, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_dense_ffn(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(out), p, n,
                               _stream(stream)))


def moe_combine(desc, y_disp, token_slot, topk_w, dense_out, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), _ptr(y_disp), _ptr(token_slot), _ptr(topk_w), _ptr(dense_out),
                             _ptr(y), _stream(stream)))


def moe_layer_forward(desc, weights: LayerWeights, x, y, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_layer_forward(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(y), p, n,
                                   _stream(stream)))


NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def moe_layer_forward_noalloc(desc, weights: LayerWeights, x, y, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(y),
                                           _stream(stream)))


def moe_layer_forward_ex(desc, weights: LayerWeights, x, y, ws, stream=None, events: Optional[PhaseEvents] = None):
    p, n = _ws(ws)
    _check(lib().moe_layer_forward_ex(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), _ptr(y), p, n,
                                      _stream(stream), ctypes.byref(events) if events is not None else None))


class ExpertStore:
    """moe_expert_store_t: every local expert in pinned host memory, `slots` of them
    cached in device slots (argument marshalling only; the store is native)."""

    def __init__(self, shape, slots: int):
        self.shape = shape
        self.desc = desc_from_shape(shape)
        h = ctypes.c_void_p()
        _check(lib().moe_expert_store_create(ctypes.byref(self.desc), int(slots), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _check(lib().moe_expert_store_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_expert(self, e: int, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: torch.Tensor):
        """Local expert e's weights from host tensors (contiguous, the layer's dtype)."""
        ts = [t.detach().to("cpu").contiguous() for t in (w1, b1, w2, b2)]
        _check(lib().moe_expert_store_set_expert(self.handle, int(e), *[t.data_ptr() for t in ts]))

    def fill(self, weights: dict):
        """All local experts from a weights dict of [E_loc, ...] tensors."""
        for i in range(self.shape.E_loc):
            self.set_expert(i, weights["w1"][i], weights["b1"][i], weights["w2"][i], weights["b2"][i])

    def weights(self, weights: dict) -> LayerWeights:
        """A LayerWeights with the gate / dense MLP of `weights` and the store's expert tables."""
        cw = make_weights({k: v for k, v in weights.items() if k not in ("w1", "b1", "w2", "b2")})
        _check(lib().moe_expert_store_weights(self.handle, ctypes.byref(cw)))
        return cw

    def update(self, demand, stream=None) -> int:
        """Fold a host int32 demand vector [E] into the scores; returns experts copied."""
        d = np.ascontiguousarray(np.asarray(demand, dtype=np.int32))
        if d.shape != (self.shape.E,):
            raise ValueError("demand must have one entry per global expert")
        n = ctypes.c_int32(0)
        _check(lib().moe_expert_store_update(self.handle, d.ctypes.data, _stream(stream), ctypes.byref(n)))
        return n.value

    def update_async(self, demand, copy_stream, stream=None) -> int:
        """The same choice with the copies on copy_stream (see commit); returns experts copied."""
        d = np.ascontiguousarray(np.asarray(demand, dtype=np.int32))
        if d.shape != (self.shape.E,):
            raise ValueError("demand must have one entry per global expert")
        n = ctypes.c_int32(0)
        _check(lib().moe_expert_store_update_async(self.handle, d.ctypes.data, _stream(stream), _stream(copy_stream),
                                                   ctypes.byref(n)))
        return n.value

    def commit(self, stream=None) -> None:
        """stream waits for the copies of a pending update_async; the copied experts switch to their slots."""
        _check(lib().moe_expert_store_commit(self.handle, _stream(stream)))

    def residency(self) -> np.ndarray:
        out = np.zeros(self.shape.E_loc, dtype=np.int32)
        _check(lib().moe_expert_store_residency(self.handle, out.ctypes.data))
        return out


class MoELayer:
    """One layer bound to its weights and a workspace (convenience for tests and the benchmark)."""

    def __init__(self, shape, weights: dict, device="cuda", store: Optional["ExpertStore"] = None):
        self.shape = shape
        self.weights = weights
        self.store = store
        self.cw = store.weights(weights) if store is not None else make_weights(weights)
        self.desc = desc_from_shape(shape)
        self.ws = torch.empty(max(moe_workspace_size(self.desc), 16), dtype=torch.uint8, device=device)

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None,
                events: Optional[PhaseEvents] = None) -> torch.Tensor:
        if x.shape != (self.shape.T, self.shape.H):
            raise ValueError(f"x must be [{self.shape.T}, {self.shape.H}]")
        if y is None:
            y = torch.empty_like(x)
        moe_layer_forward_ex(self.desc, self.cw, x, y, self.ws, stream, events)
        return y
