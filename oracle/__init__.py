"""Python binding of the plain CPU oracle (liboracle: moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import this package.  It never imports the
HIP library package, and the HIP library never imports it.

All arrays are host numpy arrays.  Outputs of the floating-point layer
functions are float64 (the oracle's own precision); the caller rounds where
the layer defines a rounding.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
BF16, I4, I2, I8 = 1, 2, 3, 4
SIGMOID_NOAUX_TC, SOFTMAX_TOPK = 0, 1


class OracleError(RuntimeError):
    pass


class _Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("router", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("routed_scaling", ctypes.c_double),
                ("expert_dtype", ctypes.c_int32), ("act_bf16", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("shared_dtype", ctypes.c_int32),
                ("top_p", ctypes.c_double)]


class _Set(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("gate_up", ctypes.POINTER(ctypes.c_void_p)),
                ("gate_up_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("down", ctypes.POINTER(ctypes.c_void_p)),
                ("down_scale", ctypes.POINTER(ctypes.c_void_p))]


@dataclass
class Desc:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    router: int = SIGMOID_NOAUX_TC
    n_group: int = 1
    topk_group: int = 1
    routed_scaling: float = 1.0
    expert_dtype: int = I4
    act_bf16: int = 0
    n_shared: int = 0
    shared_dtype: int = BF16
    top_p: float = 0.0      # adaptive expert top-p (off unless 0 < top_p < 1)

    @staticmethod
    def from_config(cfg, expert_dtype: Optional[int] = None) -> "Desc":
        return Desc(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts,
                    top_k=cfg.top_k, router=cfg.router, n_group=cfg.n_group,
                    topk_group=cfg.topk_group, routed_scaling=float(cfg.routed_scaling),
                    expert_dtype=cfg.expert_dtype if expert_dtype is None else expert_dtype,
                    act_bf16=1 if cfg.act_dtype == BF16 else 0, n_shared=cfg.n_shared,
                    shared_dtype=cfg.shared_dtype, top_p=float(np.float32(cfg.top_p)))

    def c(self) -> _Desc:
        return _Desc(self.hidden, self.inter, self.n_experts, self.top_k, self.router,
                     self.n_group, self.topk_group, self.routed_scaling, self.expert_dtype,
                     self.act_bf16, self.n_shared, self.shared_dtype, self.top_p)


_lib = None


def lib():
    global _lib
    if _lib is None:
        # MOE_ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("MOE_ORACLE_LIB") or os.path.join(HERE, "libmoe_oracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        D, S = ctypes.POINTER(_Desc), ctypes.POINTER(_Set)
        sig = {
            "orc_decode_codes": [i32, vp, i64, vp],
            "orc_dequant_rows": [i32, vp, vp, i64, i64, i64, vp],
            "orc_logits": [D, vp, vp, i32, vp],
            "orc_select": [D, vp, vp, i32, vp, vp, vp],
            "orc_route": [D, vp, vp, vp, i32, vp, vp, vp],
            "orc_bucket": [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp],
            "orc_expert_ffn": [D, S, i32, i32, vp, vp, i32, i32, vp],
            "orc_expert_h": [D, S, i32, i32, vp, vp, i32, i32, vp, vp],
            "orc_layer_forward": [D, vp, vp, S, S, vp, i32, vp, vp, vp],
            "orc_layer_forward_per_token": [D, vp, vp, S, S, vp, i32, vp],
            "orc_layer_band": [D, vp, vp, S, S, vp, i32, dbl, vp],
            "orc_rmsnorm": [vp, i32, i32, dbl, vp],
            "orc_residual_add": [vp, vp, i64],
            "orc_set_threads": [i32],
            "orc_max_threads": [],
            "orc_decode_e4m3": [vp, i64, vp],
            "orc_requant_fp8_int4": [vp, vp, i64, i64, i32, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need a contiguous array"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def set_threads(n: int):
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


class ExpertSet:
    """Per-expert host arrays; entries may be None (never evaluated)."""

    def __init__(self, dtype: int, experts: Sequence[Optional[dict]]):
        n = len(experts)
        self.dtype = dtype
        self._keep = []
        arr = lambda: (ctypes.c_void_p * n)()
        self.gu, self.gus, self.dn, self.dns = arr(), arr(), arr(), arr()
        for i, ex in enumerate(experts):
            if ex is None:
                continue
            for tab, key in ((self.gu, "gate_up"), (self.gus, "gate_up_scale"),
                             (self.dn, "down"), (self.dns, "down_scale")):
                a = ex.get(key)
                if a is None:
                    continue
                a = np.ascontiguousarray(a)
                self._keep.append(a)
                tab[i] = a.ctypes.data
        cast = lambda t: ctypes.cast(t, ctypes.POINTER(ctypes.c_void_p))
        self.c = _Set(dtype, cast(self.gu), cast(self.gus), cast(self.dn), cast(self.dns))


def decode_codes(dtype: int, packed: np.ndarray, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int8)
    _check(lib().orc_decode_codes(dtype, _p(np.ascontiguousarray(packed)), n, _p(out)))
    return out


def dequant_rows(dtype: int, codes: np.ndarray, scales: Optional[np.ndarray], cols: int,
                 row0: int, n_rows: int) -> np.ndarray:
    out = np.empty((n_rows, cols), dtype=np.float32)
    _check(lib().orc_dequant_rows(dtype, _p(np.ascontiguousarray(codes)),
                                  _p(None if scales is None else np.ascontiguousarray(scales)),
                                  cols, row0, n_rows, _p(out)))
    return out


def logits(d: Desc, w_router, x, n_tokens) -> np.ndarray:
    z = np.empty((n_tokens, d.n_experts), dtype=np.float64)
    _check(lib().orc_logits(ctypes.byref(d.c()), _p(w_router), _p(x), n_tokens, _p(z)))
    return z


def select(d: Desc, z: np.ndarray, bias, n_tokens):
    idx = np.empty((n_tokens, d.top_k), dtype=np.int32)
    w = np.empty((n_tokens, d.top_k), dtype=np.float32)
    w64 = np.empty((n_tokens, d.top_k), dtype=np.float64)
    _check(lib().orc_select(ctypes.byref(d.c()), _p(np.ascontiguousarray(z, dtype=np.float64)),
                            _p(bias), n_tokens, _p(idx), _p(w), _p(w64)))
    return idx, w, w64


def route(d: Desc, w_router, bias, x, n_tokens):
    idx = np.empty((n_tokens, d.top_k), dtype=np.int32)
    w = np.empty((n_tokens, d.top_k), dtype=np.float32)
    w64 = np.empty((n_tokens, d.top_k), dtype=np.float64)
    if n_tokens:
        _check(lib().orc_route(ctypes.byref(d.c()), _p(w_router), _p(bias), _p(x), n_tokens,
                               _p(idx), _p(w), _p(w64)))
    return idx, w, w64


def bucket(topk_idx: np.ndarray, n_experts: int) -> dict:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = (idx.shape if idx.ndim == 2 else (idx.shape[0], 1))
    F = T * K
    out = dict(counts=np.empty(n_experts, np.int32), offsets=np.empty(n_experts + 1, np.int32),
               entries=np.empty(F, np.int32), inverse=np.empty(F, np.int32),
               active=np.empty(n_experts, np.int32), n_active=np.zeros(1, np.int32))
    _check(lib().orc_bucket(T, K, n_experts, _p(idx), _p(out["counts"]), _p(out["offsets"]),
                            _p(out["entries"]), _p(out["inverse"]), _p(out["active"]),
                            _p(out["n_active"])))
    out["n_active"] = int(out["n_active"][0])
    out["active"] = out["active"][: out["n_active"]].copy()
    return out


def expert_ffn(d: Desc, eset: ExpertSet, e: int, x, rows=None, n_rows=None, row_div=1,
               inter=None) -> np.ndarray:
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = rows.shape[0]
    y = np.empty((n_rows, d.hidden), dtype=np.float64)
    if n_rows:
        _check(lib().orc_expert_ffn(ctypes.byref(d.c()), ctypes.byref(eset.c), e,
                                    inter or d.inter, _p(x), _p(rows), n_rows, row_div, _p(y)))
    return y


def expert_h(d: Desc, eset: ExpertSet, e: int, x, rows=None, n_rows=None, row_div=1,
             inter=None, with_scale=False):
    """The expert's SwiGLU output h [n_rows][inter] in fp64, before any
    rounding; with_scale: (h, e) with e the first-order scale of the error that
    rounding the terms of g and u makes in h (a test tolerance)."""
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = rows.shape[0]
    inter = inter or d.inter
    h = np.empty((n_rows, inter), dtype=np.float64)
    es = np.empty((n_rows, inter), dtype=np.float64) if with_scale else None
    if n_rows:
        _check(lib().orc_expert_h(ctypes.byref(d.c()), ctypes.byref(eset.c), e, inter, _p(x),
                                  _p(rows), n_rows, row_div, _p(h), _p(es)))
    return (h, es) if with_scale else h


def layer_forward(d: Desc, w_router, bias, routed: ExpertSet, shared: Optional[ExpertSet], x,
                  n_tokens):
    out = np.empty((n_tokens, d.hidden), dtype=np.float64)
    idx = np.empty((n_tokens, d.top_k), dtype=np.int32)
    w = np.empty((n_tokens, d.top_k), dtype=np.float32)
    if n_tokens:
        _check(lib().orc_layer_forward(ctypes.byref(d.c()), _p(w_router), _p(bias),
                                       ctypes.byref(routed.c),
                                       ctypes.byref(shared.c) if shared else None, _p(x),
                                       n_tokens, _p(out), _p(idx), _p(w)))
    return out, idx, w


def layer_forward_per_token(d: Desc, w_router, bias, routed: ExpertSet,
                            shared: Optional[ExpertSet], x, n_tokens):
    out = np.empty((n_tokens, d.hidden), dtype=np.float64)
    if n_tokens:
        _check(lib().orc_layer_forward_per_token(ctypes.byref(d.c()), _p(w_router), _p(bias),
                                                 ctypes.byref(routed.c),
                                                 ctypes.byref(shared.c) if shared else None,
                                                 _p(x), n_tokens, _p(out)))
    return out


def layer_band(d: Desc, w_router, bias, routed: ExpertSet, shared: Optional[ExpertSet], x,
               n_tokens, window: float) -> np.ndarray:
    """Output band of the bf16 rounding of h (see moe_oracle.h): an h is
    ambiguous within window * (its error scale) of a rounding midpoint; zeros
    for f32 activations."""
    band = np.empty((n_tokens, d.hidden), dtype=np.float64)
    if n_tokens:
        _check(lib().orc_layer_band(ctypes.byref(d.c()), _p(w_router), _p(bias),
                                    ctypes.byref(routed.c),
                                    ctypes.byref(shared.c) if shared else None, _p(x),
                                    n_tokens, float(window), _p(band)))
    return band


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    _check(lib().orc_rmsnorm(_p(x), x.shape[0], x.shape[1], eps, _p(out)))
    return out


def residual_add(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    y = np.ascontiguousarray(y, dtype=np.float64)
    _check(lib().orc_residual_add(_p(x), _p(y), x.size))
    return x


# ------------------------------------------------------- convenience layer --

def expert_set_from_host_layer(hl, experts=None) -> ExpertSet:
    """ExpertSet over a gen.HostLayer's routed experts (missing ones = None)."""
    n = hl.cfg.n_experts
    wanted = set(range(n)) if experts is None else set(int(e) for e in experts)
    exs = [hl.get(e) if e in wanted else None for e in range(n)]
    dtype = next(ex["dtype"] for ex in exs if ex is not None) if wanted else hl.cfg.expert_dtype
    return ExpertSet(dtype, exs)


def shared_set_from_host_layer(hl) -> Optional[ExpertSet]:
    if hl.shared is None:
        return None
    return ExpertSet(hl.shared["dtype"], [hl.shared])


def layer_forward_host(hl, x: np.ndarray, desc: Optional[Desc] = None):
    """Route first, generate only the experts the batch selects, then run the
    batch-union layer.  Returns (out float64 [T][H], topk_idx, topk_w)."""
    d = desc or Desc.from_config(hl.cfg, expert_dtype=hl.dtype)
    T = x.shape[0]
    idx, _, _ = route(d, hl.w_router, hl.bias, x, T)
    routed = expert_set_from_host_layer(hl, np.unique(idx))
    return layer_forward(d, hl.w_router, hl.bias, routed, shared_set_from_host_layer(hl), x, T)


def layer_band_host(hl, x: np.ndarray, window: float, desc: Optional[Desc] = None):
    """layer_band for a gen.HostLayer, generating only the selected experts."""
    d = desc or Desc.from_config(hl.cfg, expert_dtype=hl.dtype)
    T = x.shape[0]
    idx, _, _ = route(d, hl.w_router, hl.bias, x, T)
    routed = expert_set_from_host_layer(hl, np.unique(idx))
    return layer_band(d, hl.w_router, hl.bias, routed, shared_set_from_host_layer(hl), x, T,
                      window)


def stack_forward_host(layers, x: np.ndarray, eps: float):
    """Pre-norm residual stack: for each layer, y = MoE(RMSNorm(x)); x = x + y.
    Returns (final x float32, per-layer inputs x_l, per-layer outputs y_l)."""
    xs, ys = [], []
    x = np.ascontiguousarray(x, dtype=np.float32)
    for hl in layers:
        xs.append(x.copy())
        xn = rmsnorm(x, eps)
        y, _, _ = layer_forward_host(hl, xn)
        ys.append(y)
        x = residual_add(x, y)
    return x, xs, ys


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 bytes, as float64."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _check(lib().orc_decode_e4m3(_p(b), b.size, _p(out)))
    return out


def requant_fp8_int4(fp8: np.ndarray, block_scales: np.ndarray, block: int = 128):
    """FP8 [rows][cols] with block scales -> (packed int4 codes [rows][cols/2],
    fp32 per-row scales [rows])."""
    fp8 = np.ascontiguousarray(fp8, dtype=np.uint8)
    rows, cols = fp8.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    _check(lib().orc_requant_fp8_int4(_p(fp8), _p(np.ascontiguousarray(block_scales, np.float32)),
                                      rows, cols, block, _p(codes), _p(scales)))
    return codes, scales
