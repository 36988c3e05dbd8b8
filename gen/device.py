"""Device-resident synthetic layers in the layout the C ABI expects.

Each routed expert set is one torch uint8 tensor [n_experts][blob_stride]:
an expert is one contiguous blob (gate/up codes | down codes | gate/up scales |
down scales), like the one-read-per-expert container of the pages ("iliria"
README, "Project status": each expert is one coalesced read, the scales a
0.22% tail).  bf16 experts hold (gate/up | down) only.  Integer codes and
scales are generated in place by the device twin of the generator (bit-identical
to the host generator); bf16 weights, the router and activations are generated
on the host and copied.  Input preparation only -- no layer arithmetic here.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import (BF16, I2, I4, I8, SCALE_LO, SCALE_WIDTH, T_DN_CODES, T_DN_I8, T_DN_SCALES,
               T_GU_CODES, T_GU_I8, T_GU_SCALES, Config, HostLayer, expert, expert_bytes, router,
               scale_mult)

HERE = os.path.dirname(os.path.abspath(__file__))
_dev = None


def dev_lib():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libmoe_gen_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, i64, u64, dbl = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_double)
        L.gen_dev_fill_int4_set.argtypes = [vp, i64, i32, i64, u64, i32, i32, i32, vp]
        L.gen_dev_fill_scales_set.argtypes = [vp, i64, i32, i64, u64, i32, i32, i32, dbl, dbl,
                                              dbl, vp]
        L.gen_dev_int2_from_int4_set.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i32, i64,
                                                 i64, vp]
        L.gen_dev_fill_int8_set.argtypes = [vp, i64, i32, i64, u64, i32, i32, i32, vp]
        for f in (L.gen_dev_fill_int4_set, L.gen_dev_fill_scales_set,
                  L.gen_dev_int2_from_int4_set, L.gen_dev_fill_int8_set):
            f.restype = ctypes.c_int
        _dev = L
    return _dev


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def blob_layout(dtype: int, hidden: int, inter: int) -> dict:
    eb = expert_bytes(dtype, hidden, inter)
    gu, dn = eb["gate_up"], eb["down"]
    lay = dict(gate_up=0, down=gu, bytes=eb["total"])
    if dtype != BF16:
        lay["gate_up_scale"] = gu + dn
        lay["down_scale"] = gu + dn + 4 * 2 * inter
    lay["stride"] = (eb["total"] + 255) // 256 * 256
    return lay


@dataclass
class DeviceLayer:
    """Device tensors of one layer plus the descriptor fields."""
    cfg: Config
    expert_dtype: int
    w_router: object
    bias: Optional[object]
    routed: object                   # uint8 [E][stride]
    routed_layout: dict
    shared: Optional[object] = None  # uint8 [1][stride]
    shared_layout: Optional[dict] = None
    keep: list = field(default_factory=list)

    @property
    def desc_spec(self):
        c = self.cfg

        class _S:
            pass
        s = _S()
        for k in ("hidden", "inter", "n_experts", "top_k", "router", "n_group", "topk_group",
                  "routed_scaling", "act_dtype", "n_shared", "shared_dtype", "top_p"):
            setattr(s, k, getattr(c, k))
        s.expert_dtype = self.expert_dtype
        s.norm_eps = c.norm_eps or 0.0
        return s

    @staticmethod
    def _set(t, lay) -> dict:
        base = t.data_ptr()
        p = dict(gate_up=base + lay["gate_up"], gate_up_stride=lay["stride"],
                 down=base + lay["down"], down_stride=lay["stride"])
        if "gate_up_scale" in lay:
            p.update(gate_up_scale=base + lay["gate_up_scale"], gate_up_scale_stride=lay["stride"],
                     down_scale=base + lay["down_scale"], down_scale_stride=lay["stride"])
        return p

    def pointers(self) -> dict:
        return dict(w_router=self.w_router.data_ptr(),
                    bias=self.bias.data_ptr() if self.bias is not None else None,
                    routed=self._set(self.routed, self.routed_layout),
                    shared=self._set(self.shared, self.shared_layout) if self.shared is not None else None)

    def routed_bytes_per_expert(self) -> int:
        return self.routed_layout["bytes"]


def _host_blob(ex: dict, lay: dict) -> np.ndarray:
    b = np.zeros(lay["stride"], dtype=np.uint8)
    put = lambda off, a: b.__setitem__(slice(off, off + a.nbytes), np.ascontiguousarray(a).view(np.uint8).ravel())
    put(lay["gate_up"], ex["gate_up"])
    put(lay["down"], ex["down"])
    if "gate_up_scale" in lay:
        put(lay["gate_up_scale"], ex["gate_up_scale"])
        put(lay["down_scale"], ex["down_scale"])
    return b


def _upload(arr: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def _shared_device(cfg: Config, layer: int, device, host_shared: Optional[dict] = None):
    if cfg.n_shared == 0:
        return None, None
    I_sh = cfg.inter * cfg.n_shared
    lay = blob_layout(cfg.shared_dtype, cfg.hidden, I_sh)
    ex = host_shared if host_shared is not None else expert(cfg, layer, 0, shared=True)
    return _upload(_host_blob(ex, lay)[None, :], device), lay


def upload_host_layer(hl: HostLayer, device) -> DeviceLayer:
    """Copy a host layer (all routed experts generated on the host) to the device."""
    cfg = hl.cfg
    dtype = hl.dtype if hl.dtype is not None else cfg.expert_dtype
    lay = blob_layout(dtype, cfg.hidden, cfg.inter)
    blobs = np.stack([_host_blob(hl.get(e), lay) for e in range(cfg.n_experts)])
    sh, sh_lay = _shared_device(cfg, hl.layer, device, hl.shared)
    return DeviceLayer(cfg=cfg, expert_dtype=dtype, w_router=_upload(hl.w_router, device),
                       bias=_upload(hl.bias, device) if hl.bias is not None else None,
                       routed=_upload(blobs, device), routed_layout=lay, shared=sh,
                       shared_layout=sh_lay)


def _fill_int4_blobs(cfg: Config, layer: int, t, lay: dict, stream: int):
    L = dev_lib()
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    base = t.data_ptr()
    _check(L.gen_dev_fill_int4_set(base + lay["gate_up"], lay["stride"], E, 2 * I * H // 2,
                                   cfg.seed, layer, T_GU_CODES, 0, stream), "int4 gate/up codes")
    _check(L.gen_dev_fill_int4_set(base + lay["down"], lay["stride"], E, H * I // 2, cfg.seed,
                                   layer, T_DN_CODES, 0, stream), "int4 down codes")
    _check(L.gen_dev_fill_scales_set(base + lay["gate_up_scale"], lay["stride"], E, 2 * I,
                                     cfg.seed, layer, T_GU_SCALES, 0, SCALE_LO, SCALE_WIDTH,
                                     scale_mult(cfg, H), stream), "gate/up scales")
    _check(L.gen_dev_fill_scales_set(base + lay["down_scale"], lay["stride"], E, H, cfg.seed,
                                     layer, T_DN_SCALES, 0, SCALE_LO, SCALE_WIDTH,
                                     scale_mult(cfg, I), stream), "down scales")


def generate_device_layer(cfg: Config, layer: int, device, dtype: Optional[int] = None,
                          also_int2: bool = False):
    """Generate a layer in HBM.  int4/int2 routed experts are generated in
    place by the device twin; bf16 routed experts, the shared expert and the
    router come from the host generator.  With also_int2, returns
    (int4 layer, int2 layer) sharing router and shared expert."""
    import torch
    dtype = cfg.expert_dtype if dtype is None else dtype
    if cfg.full_codes:
        raise ValueError("full-range codes are generated on the host: use upload_host_layer")
    stream = torch.cuda.current_stream(device).cuda_stream
    w, b = router(cfg, layer)
    w_t = _upload(w, device)
    b_t = _upload(b, device) if b is not None else None
    sh, sh_lay = _shared_device(cfg, layer, device)
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    if dtype == BF16:
        lay = blob_layout(BF16, H, I)
        blobs = np.stack([_host_blob(expert(cfg, layer, e, BF16), lay) for e in range(E)])
        return DeviceLayer(cfg, BF16, w_t, b_t, _upload(blobs, device), lay, sh, sh_lay)
    if dtype == I8:
        lay = blob_layout(I8, H, I)
        t8 = torch.empty((E, lay["stride"]), dtype=torch.uint8, device=device)
        L = dev_lib()
        base = t8.data_ptr()
        _check(L.gen_dev_fill_int8_set(base + lay["gate_up"], lay["stride"], E, 2 * I * H,
                                       cfg.seed, layer, T_GU_I8, 0, stream), "int8 gate/up codes")
        _check(L.gen_dev_fill_int8_set(base + lay["down"], lay["stride"], E, H * I, cfg.seed,
                                       layer, T_DN_I8, 0, stream), "int8 down codes")
        _check(L.gen_dev_fill_scales_set(base + lay["gate_up_scale"], lay["stride"], E, 2 * I,
                                         cfg.seed, layer, T_GU_SCALES, 0, SCALE_LO, SCALE_WIDTH,
                                         scale_mult(cfg, H) / 16.0, stream), "gate/up scales")
        _check(L.gen_dev_fill_scales_set(base + lay["down_scale"], lay["stride"], E, H, cfg.seed,
                                         layer, T_DN_SCALES, 0, SCALE_LO, SCALE_WIDTH,
                                         scale_mult(cfg, I) / 16.0, stream), "down scales")
        return DeviceLayer(cfg, I8, w_t, b_t, t8, lay, sh, sh_lay)
    lay4 = blob_layout(I4, H, I)
    t4 = torch.empty((E, lay4["stride"]), dtype=torch.uint8, device=device)
    _fill_int4_blobs(cfg, layer, t4, lay4, stream)
    l4 = DeviceLayer(cfg, I4, w_t, b_t, t4, lay4, sh, sh_lay)
    if dtype == I4 and not also_int2:
        return l4
    lay2 = blob_layout(I2, H, I)
    t2 = torch.empty((E, lay2["stride"]), dtype=torch.uint8, device=device)
    L = dev_lib()
    b4, b2 = t4.data_ptr(), t2.data_ptr()
    _check(L.gen_dev_int2_from_int4_set(b4 + lay4["gate_up"], lay4["stride"],
                                        b4 + lay4["gate_up_scale"], lay4["stride"],
                                        b2 + lay2["gate_up"], lay2["stride"],
                                        b2 + lay2["gate_up_scale"], lay2["stride"], E, 2 * I, H,
                                        stream), "int2 gate/up")
    _check(L.gen_dev_int2_from_int4_set(b4 + lay4["down"], lay4["stride"],
                                        b4 + lay4["down_scale"], lay4["stride"],
                                        b2 + lay2["down"], lay2["stride"],
                                        b2 + lay2["down_scale"], lay2["stride"], E, H, I,
                                        stream), "int2 down")
    l2 = DeviceLayer(cfg, I2, w_t, b_t, t2, lay2, sh, sh_lay)
    if also_int2:
        return l4, l2
    del t4
    l2.routed_layout = lay2
    return l2
