"""Seeded synthetic inputs for the routed MoE layer workloads.

This module is shared by the oracle side and the HIP side of the tests and
the benchmark.  It holds shapes, seeds and value distributions only -- none
of the layer's arithmetic.  Every value is a pure function of
(seed, layer, tensor, expert, index) through the counter-based SplitMix64
draws in gen_core.h; the device twin (libmoe_gen_dev.so) reproduces the
integer codes and scales bit for bit, so the large expert sets can be built
in place in HBM while the oracle regenerates only the experts it evaluates.

Workloads (shapes from the pages: 256 experts per layer, top-8, about
19 MB per int4 expert -- "colibri" README, "The idea"; a Granite MoE layer --
"Glacial" page):
  c0  tiny layer, 1 token, int4 experts + int4 shared expert
  c1  Granite-shaped stack: 24 layers, bf16 experts, softmax top-8 of 32
  c2  GLM-scale decode layer, 1 token, int4 experts + bf16 shared expert
  c3  GLM-scale batch-union prefill, 2048 tokens, bf16 activations,
      Zipf-skewed expert popularity
  c4  8 stacked GLM-scale layers, batches 2/4/16, int4 and int2 variants
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# dtype codes (match the enum values used at both library boundaries)
F32, BF16, I4, I2, I8 = 0, 1, 2, 3, 4
SIGMOID_NOAUX_TC, SOFTMAX_TOPK = 0, 1

# tensor ids of gen_core.h
T_X, T_WROUTER, T_BIAS, T_GU_CODES, T_GU_SCALES, T_DN_CODES, T_DN_SCALES = 0, 1, 2, 3, 4, 5, 6
T_GU_BF16, T_DN_BF16, T_ZIPF_PERM, T_GU_I8, T_DN_I8 = 7, 8, 9, 10, 11
T_GU_BYTES, T_DN_BYTES = 12, 13

SCALE_LO, SCALE_WIDTH = 0.01, 0.04   # per-row scales U(0.01, 0.05)


@dataclass(frozen=True)
class Config:
    name: str
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    router: int
    n_group: int
    topk_group: int
    routed_scaling: float
    n_shared: int
    expert_dtype: int
    shared_dtype: int
    act_dtype: int
    n_layers: int
    batches: tuple
    seed: int
    bias: Optional[str]            # None | "normal" | "zipf"
    bias_std: float = 0.01
    scale_fanin: bool = False      # multiply scales by sqrt(64 / fan_in)
    norm_eps: Optional[float] = None
    bf16_std: float = 0.02
    zipf_s: float = 1.1
    zipf_lambda: float = 0.0
    top_p: float = 0.0             # adaptive expert top-p (0: off)
    full_codes: bool = False       # integer codes as uniform bytes: the whole range of
                                   # each container (int4 [-8, 7], int2 [-2, 1], int8
                                   # [-128, 127]) instead of the symmetric draws


# Router bias of the Zipf-skewed workload, by popularity rank: calibrated once
# on the prefill batch by oracle/calibrate_zipf_bias.py (see there) and stored
# as data; expert e of a layer takes the entry of its rank in that layer's
# seeded rank permutation.
ZIPF_BIAS_FILE = os.path.join(HERE, "zipf_bias.json")
_zipf_bias_cache = {}


def zipf_bias_by_rank(n_experts: int, top_k: int, s: float) -> Optional[np.ndarray]:
    import json
    key = (n_experts, top_k, s)
    if key not in _zipf_bias_cache:
        val = None
        if os.path.exists(ZIPF_BIAS_FILE):
            with open(ZIPF_BIAS_FILE) as f:
                doc = json.load(f)
            if (doc["n_experts"], doc["top_k"], doc["s"]) == key:
                val = np.asarray(doc["bias_by_rank"], dtype=np.float32)
        _zipf_bias_cache[key] = val
    return _zipf_bias_cache[key]


_GLM = dict(hidden=6144, inter=2048, n_experts=256, top_k=8, router=SIGMOID_NOAUX_TC,
            n_group=8, topk_group=4, routed_scaling=2.5, n_shared=1, expert_dtype=I4,
            shared_dtype=BF16, scale_fanin=True)

CONFIGS = {
    "c0": Config(name="tiny_layer_1tok", hidden=64, inter=32, n_experts=8, top_k=2,
                 router=SIGMOID_NOAUX_TC, n_group=2, topk_group=1, routed_scaling=2.5,
                 n_shared=1, expert_dtype=I4, shared_dtype=I4, act_dtype=F32, n_layers=1,
                 batches=(1,), seed=0, bias="normal"),
    "c1": Config(name="granite_stack_24x_decode", hidden=1024, inter=512, n_experts=32,
                 top_k=8, router=SOFTMAX_TOPK, n_group=1, topk_group=1, routed_scaling=1.0,
                 n_shared=0, expert_dtype=BF16, shared_dtype=BF16, act_dtype=F32,
                 n_layers=24, batches=(1,), seed=1, bias=None, norm_eps=1e-6),
    "c2": Config(name="glm_layer_decode_1tok", act_dtype=F32, n_layers=1, batches=(1,),
                 seed=2, bias="normal", **_GLM),
    "c3": Config(name="glm_layer_prefill_2048tok_zipf", act_dtype=BF16, n_layers=1,
                 batches=(2048,), seed=3, bias="zipf", **_GLM),
    "c4": Config(name="glm_stack_8x_verify", act_dtype=F32, n_layers=8, batches=(2, 4, 16),
                 seed=4, bias="normal", norm_eps=1e-6, **_GLM),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def shrink(cfg: Config, **kw) -> Config:
    """A smaller variant of a workload with the same structure (for tests)."""
    return replace(cfg, **kw)


# ------------------------------------------------------------ byte sizes --

def row_bytes(dtype: int, cols: int) -> int:
    if dtype == I4:
        return cols // 2
    if dtype == I2:
        return cols // 4
    if dtype == I8:
        return cols
    if dtype == BF16:
        return cols * 2
    if dtype == F32:
        return cols * 4
    raise ValueError(dtype)


def expert_bytes(dtype: int, hidden: int, inter: int) -> dict:
    """Bytes of one expert: gate/up codes, down codes, and their fp32 scales."""
    gu = 2 * inter * row_bytes(dtype, hidden)
    dn = hidden * row_bytes(dtype, inter)
    sc = 0 if dtype == BF16 else 4 * (2 * inter + hidden)
    return dict(gate_up=gu, down=dn, scales=sc, total=gu + dn + sc)


def scale_mult(cfg: Config, fan_in: int) -> float:
    return math.sqrt(64.0 / fan_in) if cfg.scale_fanin else 1.0


# --------------------------------------------------------- host library --

_host = None


def host_lib():
    global _host
    if _host is None:
        # MOE_GEN_LIB lets the sanitizer test load an instrumented build
        path = os.environ.get("MOE_GEN_LIB") or os.path.join(HERE, "libmoe_gen.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        i32, i64, u64, dbl, vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.gen_fill_int4.argtypes = [vp, u64, i32, i32, i32, i64]
        lib.gen_fill_scales.argtypes = [vp, u64, i32, i32, i32, i64, dbl, dbl, dbl]
        lib.gen_fill_normal_f32.argtypes = [vp, i64, u64, i32, i32, i32, dbl]
        lib.gen_fill_normal_bf16.argtypes = [vp, i64, u64, i32, i32, i32, dbl]
        lib.gen_fill_u64.argtypes = [vp, i64, u64, i32, i32, i32]
        lib.gen_int2_from_int4.argtypes = [vp, vp, i64, i64, vp, vp]
        lib.gen_fill_int8.argtypes = [vp, u64, i32, i32, i32, i64]
        lib.gen_fill_bytes.argtypes = [vp, u64, i32, i32, i32, i64]
        for fn in (lib.gen_fill_int4, lib.gen_fill_scales, lib.gen_fill_normal_f32,
                   lib.gen_fill_normal_bf16, lib.gen_fill_u64, lib.gen_int2_from_int4,
                   lib.gen_fill_int8, lib.gen_fill_bytes):
            fn.restype = None
        _host = lib
    return _host


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def int4_codes(seed, layer, tensor, expert, rows, cols) -> np.ndarray:
    out = np.empty((rows, cols // 2), dtype=np.uint8)
    host_lib().gen_fill_int4(_p(out), seed, layer, tensor, expert, out.size)
    return out


def int8_codes(seed, layer, tensor, expert, rows, cols) -> np.ndarray:
    """int8 codes uniform on {-127..127}, row-major [rows][cols] bytes."""
    out = np.empty((rows, cols), dtype=np.uint8)
    host_lib().gen_fill_int8(_p(out), seed, layer, tensor, expert, out.size)
    return out


def code_bytes(seed, layer, tensor, expert, rows, row_bytes) -> np.ndarray:
    """Uniform bytes [rows][row_bytes]: packed codes over a container's whole range."""
    out = np.empty((rows, row_bytes), dtype=np.uint8)
    host_lib().gen_fill_bytes(_p(out), seed, layer, tensor, expert, out.size)
    return out


def int8_from_int4(codes4: np.ndarray, cols: int) -> np.ndarray:
    """The int8 container holding the same codes as a packed int4 matrix
    (each nibble sign-extended to a byte)."""
    b = np.ascontiguousarray(codes4, dtype=np.uint8).reshape(-1, cols // 2)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((b.shape[0], cols), dtype=np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out.astype(np.int8).view(np.uint8)


def expert_i8_from_i4(ex: dict, hidden: int, inter: int) -> dict:
    """An int4 expert re-packed into the int8 container (same codes, same
    scales)."""
    assert ex["dtype"] == I4
    return dict(dtype=I8, gate_up=int8_from_int4(ex["gate_up"], hidden),
                gate_up_scale=ex["gate_up_scale"], down=int8_from_int4(ex["down"], inter),
                down_scale=ex["down_scale"])


def scales(seed, layer, tensor, expert, rows, mult) -> np.ndarray:
    out = np.empty(rows, dtype=np.float32)
    host_lib().gen_fill_scales(_p(out), seed, layer, tensor, expert, rows, SCALE_LO,
                               SCALE_WIDTH, mult)
    return out


def normal_f32(shape, seed, layer, tensor, expert, std) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    host_lib().gen_fill_normal_f32(_p(out), out.size, seed, layer, tensor, expert, std)
    return out


def normal_bf16(shape, seed, layer, tensor, expert, std) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, std^2) draws rounded float -> bf16."""
    out = np.empty(shape, dtype=np.uint16)
    host_lib().gen_fill_normal_bf16(_p(out), out.size, seed, layer, tensor, expert, std)
    return out


def u64_draws(n, seed, layer, tensor, expert) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    host_lib().gen_fill_u64(_p(out), n, seed, layer, tensor, expert)
    return out


def int2_from_int4(codes4: np.ndarray, s4: np.ndarray, cols: int):
    rows = codes4.shape[0]
    c2 = np.empty((rows, cols // 4), dtype=np.uint8)
    s2 = np.empty(rows, dtype=np.float32)
    host_lib().gen_int2_from_int4(_p(np.ascontiguousarray(codes4)), _p(np.ascontiguousarray(s4)),
                                  rows, cols, _p(c2), _p(s2))
    return c2, s2


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ------------------------------------------------------------- host sets --

def x_tokens(cfg: Config, n_tokens: int, batch_id: int = 0, layer: int = 0) -> np.ndarray:
    """Activations x ~ N(0,1): float32 [T][H], or bf16 bits [T][H] when the
    workload's activations are bf16 (rounded float -> bf16)."""
    if cfg.act_dtype == BF16:
        return normal_bf16((n_tokens, cfg.hidden), cfg.seed, layer, T_X, batch_id, 1.0)
    return normal_f32((n_tokens, cfg.hidden), cfg.seed, layer, T_X, batch_id, 1.0)


def zipf_targets(n_experts: int, top_k: int, s: float) -> np.ndarray:
    """Per-token selection probability of popularity rank r (1-based):
    P_r = min(1, c r^-s) with sum_r P_r = top_k (c by bisection)."""
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    lo, hi = 0.0, float(n_experts)
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * r ** (-s)).sum() < top_k:
            lo = c
        else:
            hi = c
    return np.minimum(1.0, 0.5 * (lo + hi) * r ** (-s))


def zipf_ranks(cfg: Config, layer: int = 0) -> np.ndarray:
    """rank[e] (1-based popularity rank of expert e) from a seeded permutation."""
    d = u64_draws(cfg.n_experts, cfg.seed, layer, T_ZIPF_PERM, 0)
    order = np.argsort(d, kind="stable")          # order[r-1] = expert of rank r
    rank = np.empty(cfg.n_experts, dtype=np.int64)
    rank[order] = np.arange(1, cfg.n_experts + 1)
    return rank


def router(cfg: Config, layer: int = 0):
    """(W_r float32 [E][H] ~ N(0, 1/H), bias float32 [E] or None)."""
    w = normal_f32((cfg.n_experts, cfg.hidden), cfg.seed, layer, T_WROUTER, 0,
                   1.0 / math.sqrt(cfg.hidden))
    if cfg.bias is None:
        return w, None
    if cfg.bias == "normal":
        return w, normal_f32((cfg.n_experts,), cfg.seed, layer, T_BIAS, 0, cfg.bias_std)
    if cfg.bias == "zipf":
        rank = zipf_ranks(cfg, layer)
        table = zipf_bias_by_rank(cfg.n_experts, cfg.top_k, cfg.zipf_s)
        if table is None or cfg.zipf_lambda:
            # no calibration for this shape: a log-popularity bias of strength
            # zipf_lambda (0.25 unless set) keeps the skew qualitatively
            lam = cfg.zipf_lambda or 0.25
            p = zipf_targets(cfg.n_experts, cfg.top_k, cfg.zipf_s)
            return w, (lam * np.log(p[rank - 1])).astype(np.float32)
        return w, table[rank - 1].copy()
    raise ValueError(cfg.bias)


def expert(cfg: Config, layer: int, e: int, dtype: Optional[int] = None, shared: bool = False):
    """Host copy of one expert: dict(gate_up, gate_up_scale, down, down_scale).

    Routed experts use expert index e; the shared expert uses index n_experts
    (its own streams).  int2 experts are derived from the int4 ones; int8
    experts draw full-range codes from their own streams, with the int4 scale
    streams divided by 16 (weights of similar magnitude).
    """
    H = cfg.hidden
    I = cfg.inter * (cfg.n_shared if shared else 1)
    if dtype is None:
        dtype = cfg.shared_dtype if shared else cfg.expert_dtype
    eid = cfg.n_experts if shared else e
    if cfg.full_codes and dtype in (I4, I2, I8):
        ppb = {I4: 2, I2: 4, I8: 1}[dtype]
        mult = 1.0 / 16.0 if dtype == I8 else 1.0
        gu = code_bytes(cfg.seed, layer, T_GU_BYTES, eid, 2 * I, H // ppb)
        dn = code_bytes(cfg.seed, layer, T_DN_BYTES, eid, H, I // ppb)
        gus = scales(cfg.seed, layer, T_GU_SCALES, eid, 2 * I, scale_mult(cfg, H) * mult)
        dns = scales(cfg.seed, layer, T_DN_SCALES, eid, H, scale_mult(cfg, I) * mult)
        return dict(dtype=dtype, gate_up=gu, gate_up_scale=gus, down=dn, down_scale=dns)
    if dtype == I8:
        gu = int8_codes(cfg.seed, layer, T_GU_I8, eid, 2 * I, H)
        gus = scales(cfg.seed, layer, T_GU_SCALES, eid, 2 * I, scale_mult(cfg, H) / 16.0)
        dn = int8_codes(cfg.seed, layer, T_DN_I8, eid, H, I)
        dns = scales(cfg.seed, layer, T_DN_SCALES, eid, H, scale_mult(cfg, I) / 16.0)
        return dict(dtype=I8, gate_up=gu, gate_up_scale=gus, down=dn, down_scale=dns)
    if dtype == BF16:
        gu = normal_bf16((2 * I, H), cfg.seed, layer, T_GU_BF16, eid, cfg.bf16_std)
        dn = normal_bf16((H, I), cfg.seed, layer, T_DN_BF16, eid, cfg.bf16_std)
        return dict(dtype=BF16, gate_up=gu, gate_up_scale=None, down=dn, down_scale=None)
    gu = int4_codes(cfg.seed, layer, T_GU_CODES, eid, 2 * I, H)
    gus = scales(cfg.seed, layer, T_GU_SCALES, eid, 2 * I, scale_mult(cfg, H))
    dn = int4_codes(cfg.seed, layer, T_DN_CODES, eid, H, I)
    dns = scales(cfg.seed, layer, T_DN_SCALES, eid, H, scale_mult(cfg, I))
    if dtype == I4:
        return dict(dtype=I4, gate_up=gu, gate_up_scale=gus, down=dn, down_scale=dns)
    if dtype == I2:
        gu2, gus2 = int2_from_int4(gu, gus, H)
        dn2, dns2 = int2_from_int4(dn, dns, I)
        return dict(dtype=I2, gate_up=gu2, gate_up_scale=gus2, down=dn2, down_scale=dns2)
    raise ValueError(dtype)


@dataclass
class HostLayer:
    cfg: Config
    layer: int
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    experts: dict = field(default_factory=dict)   # e -> expert dict (lazily filled)
    shared: Optional[dict] = None
    dtype: Optional[int] = None

    def get(self, e: int) -> dict:
        if e not in self.experts:
            self.experts[e] = expert(self.cfg, self.layer, e, self.dtype)
        return self.experts[e]


def host_layer(cfg: Config, layer: int = 0, experts=None, dtype: Optional[int] = None) -> HostLayer:
    """Router, shared expert and (optionally) a subset of routed experts on the
    host; other experts are generated on first use through HostLayer.get."""
    w, b = router(cfg, layer)
    hl = HostLayer(cfg=cfg, layer=layer, w_router=w, bias=b, dtype=dtype)
    if cfg.n_shared > 0:
        hl.shared = expert(cfg, layer, 0, shared=True)
    for e in (range(cfg.n_experts) if experts == "all" else (experts or [])):
        hl.get(e)
    return hl


# ---------------------------------------------------------- FP8 inputs --

def fp8_e4m3_matrix(seed: int, rows: int, cols: int, block: int = 128, kind: str = "normal"):
    """A synthetic FP8 checkpoint matrix: OCP E4M3 bytes [rows][cols] and fp32
    block scales [ceil(rows/block)][ceil(cols/block)].  kind "normal": weights
    N(0, 1) rounded to E4M3 (torch's conversion), the shape of a real FP8
    checkpoint; kind "bytes": every non-NaN byte value, uniformly."""
    rng = np.random.default_rng([seed, rows, cols, block])
    if kind == "bytes":
        b = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        b[(b & 0x7F) == 0x7F] = 0x00
    else:
        import torch
        v = rng.standard_normal((rows, cols)).astype(np.float32)
        b = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    nb_r, nb_c = -(-rows // block), -(-cols // block)
    bs = rng.uniform(2.0 ** -12, 2.0 ** -6, size=(nb_r, nb_c)).astype(np.float32)
    return b, bs
