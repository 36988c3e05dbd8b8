"""ctypes binding of libmoe.so (include/moe.h): argument marshalling only.

Functions named moe_* mirror the C ABI one to one: they take ctypes
structures, device pointers (ints or torch tensors) and a stream handle, and
raise MoeError on a non-OK status.  PyTorch is used only to own device memory
and streams.  Every computation runs in the HIP kernels of libmoe.so; if the
library is missing this module raises on first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20
MOE_F32, MOE_BF16, MOE_I4, MOE_I2 = 0, 1, 2, 3
MOE_ROUTER_SIGMOID_NOAUX_TC, MOE_ROUTER_SOFTMAX_TOPK = 0, 1
(MOE_STAGE_ROUTE, MOE_STAGE_BUCKET, MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_COMBINE,
 MOE_N_STAGES) = range(6)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)}")
        self.status = status


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("router", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("routed_scaling", ctypes.c_float),
                ("expert_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("shared_dtype", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("top_p", ctypes.c_float)]


class MoeExpertSet(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("gate_up_stride", ctypes.c_int64),
                ("gate_up_scale", ctypes.c_void_p), ("gate_up_scale_stride", ctypes.c_int64),
                ("down", ctypes.c_void_p), ("down_stride", ctypes.c_int64),
                ("down_scale", ctypes.c_void_p), ("down_scale_stride", ctypes.c_int64)]


class MoeLayerWeights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("routed", MoeExpertSet), ("shared", MoeExpertSet)]


class MoeLaunchOpts(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("h_f32", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build(); "
                               "there is no fallback implementation")
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str):
    """A libmoe.so at `path` with the C ABI's signatures declared (the in-tree
    build is lib(); a benchmark A/B loads another build this way)."""
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    D = ctypes.POINTER(MoeLayerDesc)
    S = ctypes.POINTER(MoeExpertSet)
    W = ctypes.POINTER(MoeLayerWeights)
    O = ctypes.POINTER(MoeLaunchOpts)
    sig = {
        "moe_workspace_bytes": ([D, i32], sz),
        "moe_route": ([D, vp, vp, vp, i32, vp, vp, vp, sz, vp], i32),
        "moe_bucket": ([i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_expert_ffn": ([D, S, i32, i32, vp, vp, i32, i32, vp, vp, sz, vp], i32),
        "moe_layer_forward": ([D, W, vp, i32, vp, vp, vp, vp, sz, vp], i32),
        "moe_layer_forward_ex": ([D, W, vp, i32, vp, vp, vp, vp, sz, vp, O], i32),
        "moe_layer_forward_noalloc": ([D, W, vp, i32, vp, vp, vp, vp], i32),
        "moe_rmsnorm": ([vp, i32, i32, f32, vp, vp], i32),
        "moe_stack_forward": ([D, W, i32, vp, i32, vp, vp, sz, vp], i32),
        "moe_dequant_rows": ([i32, vp, vp, i32, i32, i32, vp, vp, vp], i32),
        "moe_status_str": ([i32], ctypes.c_char_p),
        "moe_requant_fp8_int4": ([vp, vp, i32, i32, i32, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _ptr(a) -> Optional[int]:
    """Device pointer of a torch tensor, an int, or None (NULL)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a if a != 0 else None
    return a.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoeError(st, where)


# ------------------------------------------------------------ raw C calls

def moe_workspace_bytes(desc: MoeLayerDesc, n_tokens: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), n_tokens))


def moe_route(desc, w_router, bias, x, n_tokens, topk_idx, topk_w, ws, ws_bytes, stream=None):
    _check(lib().moe_route(ctypes.byref(desc), _ptr(w_router), _ptr(bias), _ptr(x), n_tokens,
                           _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_route")


def moe_bucket(n_tokens, top_k, n_experts, topk_idx, counts, offsets, entries, inverse, active,
               n_active, ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_bucket(n_tokens, top_k, n_experts, _ptr(topk_idx), _ptr(counts),
                            _ptr(offsets), _ptr(entries), _ptr(inverse), _ptr(active),
                            _ptr(n_active), _ptr(ws), ws_bytes, _stream(stream)), "moe_bucket")


def moe_expert_ffn(desc, eset: MoeExpertSet, shared, expert, x, rows, n_rows, row_div, y, ws,
                   ws_bytes, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(desc), ctypes.byref(eset), shared, expert, _ptr(x),
                                _ptr(rows), n_rows, row_div, _ptr(y), _ptr(ws), ws_bytes,
                                _stream(stream)), "moe_expert_ffn")


def moe_layer_forward(desc, weights: MoeLayerWeights, x, n_tokens, out, topk_idx_out,
                      topk_w_out, ws, ws_bytes, stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(desc), ctypes.byref(weights), _ptr(x), n_tokens,
                                   _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws),
                                   ws_bytes, _stream(stream)), "moe_layer_forward")


def moe_layer_forward_ex(desc, weights: MoeLayerWeights, x, n_tokens, out, topk_idx_out,
                         topk_w_out, ws, ws_bytes, stream=None, events=None, h_f32=None):
    """events: optional list of 2*MOE_N_STAGES raw hipEvent_t handles (ints);
    h_f32: optional device buffer for the fp32 h before rounding (test hook)."""
    opts = None
    keep = None
    if events is not None or h_f32 is not None:
        evp = None
        if events is not None:
            keep = (ctypes.c_void_p * len(events))(*[e or None for e in events])
            evp = ctypes.cast(keep, ctypes.POINTER(ctypes.c_void_p))
        opts = MoeLaunchOpts(evp, _ptr(h_f32))
    _check(lib().moe_layer_forward_ex(ctypes.byref(desc), ctypes.byref(weights), _ptr(x),
                                      n_tokens, _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out),
                                      _ptr(ws), ws_bytes, _stream(stream),
                                      ctypes.byref(opts) if opts is not None else None),
           "moe_layer_forward_ex")


def moe_layer_forward_noalloc(desc, weights: MoeLayerWeights, x, n_tokens, out, topk_idx_out,
                              topk_w_out, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(weights), _ptr(x),
                                           n_tokens, _ptr(out), _ptr(topk_idx_out),
                                           _ptr(topk_w_out), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_rmsnorm(x, n_tokens, hidden, eps, out, stream=None):
    _check(lib().moe_rmsnorm(_ptr(x), n_tokens, hidden, eps, _ptr(out), _stream(stream)),
           "moe_rmsnorm")


def moe_stack_forward(desc, layers, n_layers, x, n_tokens, y_layers, ws, ws_bytes, stream=None):
    """layers: a ctypes array of MoeLayerWeights (host memory)."""
    _check(lib().moe_stack_forward(ctypes.byref(desc), layers, n_layers, _ptr(x), n_tokens,
                                   _ptr(y_layers), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_stack_forward")


def moe_dequant_rows(dtype, codes, scales, cols, row0, n_rows, out_f32, out_bf16=None,
                     stream=None):
    _check(lib().moe_dequant_rows(dtype, _ptr(codes), _ptr(scales), cols, row0, n_rows,
                                  _ptr(out_f32), _ptr(out_bf16), _stream(stream)),
           "moe_dequant_rows")


# --------------------------------------------------- marshalling helpers

def make_desc(spec) -> MoeLayerDesc:
    """MoeLayerDesc from any object with the descriptor's field names."""
    g = lambda k, dflt=None: getattr(spec, k, dflt)
    return MoeLayerDesc(hidden=g("hidden"), inter=g("inter"), n_experts=g("n_experts"),
                        top_k=g("top_k"), router=g("router"), n_group=g("n_group"),
                        topk_group=g("topk_group"), routed_scaling=g("routed_scaling"),
                        expert_dtype=g("expert_dtype"), act_dtype=g("act_dtype"),
                        n_shared=g("n_shared"), shared_dtype=g("shared_dtype"),
                        norm_eps=g("norm_eps", None) or 0.0, top_p=g("top_p", None) or 0.0)


def make_set(p: Optional[dict]) -> MoeExpertSet:
    """MoeExpertSet from a dict of device pointers (ints) and byte strides."""
    if not p:
        return MoeExpertSet()
    return MoeExpertSet(p["gate_up"], p["gate_up_stride"], p.get("gate_up_scale") or None,
                        p.get("gate_up_scale_stride", 0), p["down"], p["down_stride"],
                        p.get("down_scale") or None, p.get("down_scale_stride", 0))


def make_weights(p: dict) -> MoeLayerWeights:
    """MoeLayerWeights from dict(w_router=ptr, bias=ptr|None, routed=dict, shared=dict|None)."""
    return MoeLayerWeights(p["w_router"], p.get("bias") or None, make_set(p["routed"]),
                           make_set(p.get("shared")))


class Workspace:
    """A growable device workspace (a torch uint8 buffer)."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        import torch
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


def layer_forward(layer, x, out=None, ws: Optional[Workspace] = None, stream=None):
    """Convenience: run moe_layer_forward on a layer object exposing .desc_spec
    (descriptor fields) and .pointers() (dict for make_weights); allocates the
    outputs and workspace with torch.  Returns (out, topk_idx, topk_w)."""
    import torch
    desc = make_desc(layer.desc_spec)
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, desc.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, desc.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, desc.top_k), dtype=torch.float32, device=dev)
    ws = ws or Workspace(dev)
    buf, nbytes = ws.get(moe_workspace_bytes(desc, T))
    moe_layer_forward(desc, make_weights(layer.pointers()), x, T, out, idx, w, buf, nbytes, stream)
    return out, idx, w


def moe_requant_fp8_int4(fp8, block_scales, rows: int, cols: int, block: int, codes, scales,
                         stream=None):
    """FP8 (E4M3) [rows][cols] + block scales -> packed int4 codes + per-row scales."""
    _check(lib().moe_requant_fp8_int4(_ptr(fp8), _ptr(block_scales), rows, cols, block,
                                      _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_requant_fp8_int4")
