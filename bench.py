#!/usr/bin/env python3
"""Benchmark: routed MoE layer tokens/s and achieved HBM GB/s on one MI355X.

A step is one full pass of the routed layer (router, batch-union bucketing,
dequant-on-use expert SwiGLU, shared expert, weighted combine) over one batch
of seeded synthetic tokens, through the C ABI of libmoe.so.

Default workload (c2): the GLM-scale decode layer -- H 6144, I 2048, 256
int4 experts (per-row fp32 scales), top-8 of 8 groups keeping 4, scaling 2.5,
one bf16 shared expert -- one token per step.  Steps rotate over 8 distinct
seeded layer instances (about 39 GB of weights) and 64 distinct tokens, so
each step reads its experts, shared expert and router from HBM rather than
from the 256 MB Infinity Cache, as successive layers of a decoder would.

The timed steps are captured once into a HIP graph and replayed (the library
allocates nothing and never synchronises, so the whole step is capturable).
A second replay of the same steps carries an event pair around the gate/up
launch of every step (and around every stage with --stages), and a third an
event pair around every whole step: its median less the event-free time per
step is what a bracket adds around running kernels, and is subtracted from
the gate/up bracket.  This times the dominant kernel without putting event
nodes into the headline loop.

Output: one JSON line (see the fields below).  --gpus N > 1 exits: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Bind the process to the system ROCm runtime before torch loads its bundled
# copy (same soname): the bundled runtime rejects event records inside stream
# capture, which the graph-replayed timing below relies on.  torch then runs on
# the system runtime too; it is only used for device memory.
_SYS_HIP = "/opt/rocm/lib/libamdhip64.so.7"
if os.path.exists(_SYS_HIP) and "torch" not in sys.modules:
    ctypes.CDLL(_SYS_HIP, mode=ctypes.RTLD_GLOBAL)

import numpy as np  # noqa: E402

import gen  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
METRIC = "MoE layer tokens/s + achieved HBM GB/s (int4 decode) at 1 MI355X"


# ------------------------------------------------------------- HIP events
class Hip:
    """The few HIP runtime calls the benchmark needs (events, stream capture)."""

    def __init__(self):
        L = ctypes.CDLL("libamdhip64.so.7")
        vp, P = ctypes.c_void_p, ctypes.POINTER
        L.hipEventCreate.argtypes = [P(vp)]
        L.hipEventElapsedTime.argtypes = [P(ctypes.c_float), vp, vp]
        L.hipEventRecord.argtypes = [vp, vp]
        L.hipEventRecordWithFlags.argtypes = [vp, vp, ctypes.c_uint]
        L.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
        L.hipStreamEndCapture.argtypes = [vp, P(vp)]
        L.hipGraphInstantiate.argtypes = [P(vp), vp, vp, vp, ctypes.c_size_t]
        L.hipGraphLaunch.argtypes = [vp, vp]
        L.hipGraphUpload.argtypes = [vp, vp]
        self.L = L

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed (hipError {rc})")

    def event(self) -> int:
        e = ctypes.c_void_p()
        self._ok(self.L.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e.value

    def record(self, ev: int, stream: int, captured: bool):
        """Record ev on stream; inside a stream capture as an event-record
        node (hipEventRecordExternal), which timestamps on every replay."""
        if captured:
            self._ok(self.L.hipEventRecordWithFlags(ev, stream, 1), "hipEventRecordWithFlags")
        else:
            self._ok(self.L.hipEventRecord(ev, stream), "hipEventRecord")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self._ok(self.L.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)

    def capture(self, stream: int, fn) -> int:
        """Record fn()'s launches on `stream` into an instantiated graph."""
        self._ok(self.L.hipStreamBeginCapture(stream, 2), "hipStreamBeginCapture")  # relaxed
        try:
            fn()
        finally:
            g = ctypes.c_void_p()
            rc = self.L.hipStreamEndCapture(stream, ctypes.byref(g))
        self._ok(rc, "hipStreamEndCapture")
        ex = ctypes.c_void_p()
        self._ok(self.L.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0), "hipGraphInstantiate")
        return ex.value

    def launch(self, exe: int, stream: int):
        self._ok(self.L.hipGraphLaunch(exe, stream), "hipGraphLaunch")

    def upload(self, exe: int, stream: int):
        """Move an instantiated graph's work to the device ahead of its first
        launch (runs none of its nodes)."""
        self._ok(self.L.hipGraphUpload(exe, stream), "hipGraphUpload")


# ------------------------------------------------ counter-measured traffic
# HBM bytes per launch of the gate/up kernel on the default workload, from the
# FETCH_SIZE and WRITE_SIZE counters (rocprofv3 --pmc, one pass each) scaled by
# what the same counters read for a plain 1 GiB device copy.  The record holds
# a digest of the sources that build and launch the kernel; once any of them
# changes the counters no longer describe it and the traffic is reported null.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_gemv_gate_up__glm_layer_decode_1tok.md")
TRAFFIC_SOURCES = ["gemv_impl.h", "route_device.h", "unpack.h", "k_gemv.hip", "k_gemv_sel.hip",
                   "down_fused.h", "moe_internal.h", "moe_capi.cpp"]


def kernel_sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_expert_ffn_sigmoid_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    if workload != "c2" or not os.path.exists(TRAFFIC_RECORD):
        return None
    with open(TRAFFIC_RECORD) as f:
        for line in f:
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("sources_sha256") == kernel_sources_digest():
                    return int(rec["bytes_per_launch"])
    return None


# ------------------------------------------------------- byte accounting
def expert_bytes(cfg, dtype):
    return gen.expert_bytes(dtype, cfg.hidden, cfg.inter)


def _ring(dtype, K):
    """Whether the expert GEMV streams rows of length K of this format through
    its LDS ring (64 lanes on a row, a compiled slice length)."""
    if dtype == gen.BF16:
        return K % 512 == 0 and K // 64 in (8, 16, 32, 64, 96, 112, 128)
    if dtype in (gen.I4, gen.I8, gen.I2):
        return K % 2048 == 0 and K // 64 in (32, 64, 96, 128)
    return False


def shared_runs_with_router(cfg, dtype, T):
    """Decode layers with a shared expert run its gate/up and down launches
    together with the router (its leading blocks compute the logits, then the
    selection): sigmoid router with at most 256 experts, and ring-streamed
    rows for both sets.  The gate/up stage then holds the routed experts only."""
    Is = cfg.inter * max(cfg.n_shared, 1)
    return (T <= 16 and cfg.n_shared > 0 and cfg.router == gen.SIGMOID_NOAUX_TC
            and cfg.n_experts <= 256
            and _ring(dtype, cfg.hidden) and _ring(dtype, cfg.inter)
            and _ring(cfg.shared_dtype, cfg.hidden) and _ring(cfg.shared_dtype, Is))


def shared_down_in_gate_up(cfg, dtype, T):
    """One-token decode whose gate/up launch selects in every block (the
    integer GLM-scale layer, or a bf16 one of 1024 columns, with the router
    beside the shared expert): with a bf16 shared expert of 2048 columns the
    waves that do not select run the shared expert's down projection there."""
    sel = ((dtype in (gen.I4, gen.I8) and cfg.hidden == 96 * 64 and 192 < cfg.n_experts <= 256)
           or (dtype == gen.BF16 and cfg.hidden == 16 * 64 and cfg.n_experts <= 64))
    return (T == 1 and sel and shared_runs_with_router(cfg, dtype, T)
            and cfg.shared_dtype == gen.BF16 and cfg.inter * cfg.n_shared == 2048)


def gate_up_bytes(cfg, dtype, n_active, T):
    """Algorithmic bytes of one gate/up launch: every active expert's gate/up
    codes and scales once, the activations once, h written once; the shared
    expert's gate/up once when it shares the launch; and, when the launch
    also runs the shared expert's down projection, its weights once, its h
    read once and its output written once."""
    eb = expert_bytes(cfg, dtype)
    scale_bytes = 0 if dtype == gen.BF16 else 4 * 2 * cfg.inter
    act = 2 if cfg.act_dtype == gen.BF16 else 4
    b = n_active * (eb["gate_up"] + scale_bytes) + T * cfg.hidden * act
    b += T * cfg.top_k * cfg.inter * act
    if cfg.n_shared and not shared_runs_with_router(cfg, dtype, T):
        Is = cfg.inter * cfg.n_shared
        sb = gen.expert_bytes(cfg.shared_dtype, cfg.hidden, Is)
        b += sb["gate_up"] + (0 if cfg.shared_dtype == gen.BF16 else 4 * 2 * Is) + T * Is * act
    if shared_down_in_gate_up(cfg, dtype, T):
        Is = cfg.inter * cfg.n_shared
        b += gen.expert_bytes(cfg.shared_dtype, cfg.hidden, Is)["down"] + Is * act + cfg.hidden * 4
    return b


def gate_up_flops(cfg, T):
    """Algorithmic flops of one gate/up launch: every (token, routed expert)
    pair and every token through the shared expert, 2 flops per weight."""
    f = 2.0 * T * cfg.top_k * 2 * cfg.inter * cfg.hidden
    if cfg.n_shared:
        f += 2.0 * T * 2 * cfg.inter * cfg.n_shared * cfg.hidden
    return f


def layer_bytes(cfg, dtype, n_active, T):
    """Algorithmic bytes of one layer step: unique routed experts, shared
    expert, router weights and bias, activations in, fp32 output out."""
    b = n_active * expert_bytes(cfg, dtype)["total"]
    if cfg.n_shared:
        b += gen.expert_bytes(cfg.shared_dtype, cfg.hidden, cfg.inter * cfg.n_shared)["total"]
    b += cfg.n_experts * cfg.hidden * 4 + (cfg.n_experts * 4 if cfg.bias else 0)
    b += T * cfg.hidden * (2 if cfg.act_dtype == gen.BF16 else 4) + T * cfg.hidden * 4
    return b


# ------------------------------------------------------------ CPU oracle
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(cfg, dtype, T, seconds, max_tokens):
    import oracle
    d = oracle.Desc.from_config(cfg, expert_dtype=dtype)
    hl = gen.host_layer(cfg, 0, dtype=dtype)
    spent, done, b = 0.0, 0, 0
    while done < max_tokens:
        x = gen.x_tokens(cfg, T, batch_id=b)
        idx, _, _ = oracle.route(d, hl.w_router, hl.bias, x, T)
        routed = oracle.expert_set_from_host_layer(hl, np.unique(idx))
        shared = oracle.shared_set_from_host_layer(hl)
        t0 = time.perf_counter()
        oracle.layer_forward(d, hl.w_router, hl.bias, routed, shared, x, T)
        spent += time.perf_counter() - t0
        done += T
        b += 1
        hl.experts.clear()
        if spent >= seconds:
            break
    return done / spent, done, b, spent


def cpu_baseline(cfg, dtype, T, seconds, max_tokens=256):
    """The oracle as it stands on a bounded sample of the same workload:
    token batches of the workload, each on layer 0; only the oracle's layer
    forward is timed (expert generation on the host is not).  Timed on all
    the host threads the oracle uses, and on one."""
    import oracle
    cores = oracle.max_threads()
    rate, done, b, spent = _oracle_rate(cfg, dtype, T, seconds, max_tokens)
    oracle.set_threads(1)
    try:
        rate1, done1, b1, spent1 = _oracle_rate(cfg, dtype, T, seconds, max_tokens)
    finally:
        oracle.set_threads(cores)
    return dict(value=rate, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{done} tokens in {b} batches of {T} (layer 0 of the workload), "
                       f"oracle layer forward timed for {spent:.1f} s",
                one_thread={"value": rate1, "unit": "tokens/s", "cores": 1,
                            "sample": f"{done1} tokens in {b1} batches of {T}, "
                                      f"timed for {spent1:.1f} s"},
                cpu_model=cpu_model())


# -------------------------------------------------------- requantization
def bench_requant(args):
    """FP8 (E4M3, 128x128 block scales) -> int4 requantization of GLM-shaped
    experts (gate/up [2I][H] and down [H][I] of 16 experts, stacked), with
    the inputs resident in HBM; a step requantizes them all."""
    import torch
    from quantized_expert_ffn_sigmoid_amd import capi
    dev = torch.device("cuda:0")
    hip = Hip()
    cfg = gen.get_config("c2")
    H, I, NE, blk = cfg.hidden, cfg.inter, 16, 128
    mats = []
    for rows, cols in ((NE * 2 * I, H), (NE * H, I)):
        g = torch.Generator(device=dev).manual_seed(rows)
        fp8 = torch.randn((rows, cols), device=dev, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
        bs = torch.rand(((rows + blk - 1) // blk, (cols + blk - 1) // blk), device=dev,
                        generator=g) * 2.0 ** -6 + 2.0 ** -12
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty(rows, dtype=torch.float32, device=dev)
        mats.append((fp8, bs, rows, cols, codes, scales))
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    def step():
        for fp8, bs, rows, cols, codes, scales in mats:
            capi.moe_requant_fp8_int4(fp8, bs, rows, cols, blk, codes, scales, stream=sh)

    K, W = args.steps, args.warmup
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, sh, False)
    for _ in range(K):
        step()
    hip.record(e1, sh, False)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1) / K
    # algorithmic bytes: every FP8 byte and block scale read once, codes and
    # row scales written once
    nbytes = sum(r * c + bs.numel() * 4 + r * c // 2 + r * 4 for _, bs, r, c, _, _ in mats)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "FP8 -> int4 expert requantization (GB/s of HBM traffic)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"FP8 E4M3 with {blk}x{blk} block scales -> int4 per-row, "
                               f"{NE} GLM experts (gate/up {2 * I}x{H}, down {H}x{I})",
                   "experts_per_step": NE},
        "roofline": {"kernel": "moe::k_requant_fp8_int4", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_step": int(nbytes)},
    }
    print(json.dumps(res), flush=True)


# ------------------------------------------------------------------ main
def percentiles(v):
    v = np.asarray(v, dtype=np.float64)
    return {"median": round(float(np.median(v)), 3), "p10": round(float(np.percentile(v, 10)), 3),
            "p90": round(float(np.percentile(v, 90)), 3)}


def run_workload(args, wl, K, W, with_cpu, replays=5, ab_lib=None):
    """Build the workload's inputs in HBM, capture its steps into HIP graphs and
    time them; returns the result dict (see the fields at the end)."""
    import torch
    from gen import device as gdev
    from quantized_expert_ffn_sigmoid_amd import capi

    dev = torch.device("cuda:0")
    hip = Hip()
    base = {"c2": "c2", "c2i8": "c2", "c4i4": "c4", "c4i2": "c4", "c3": "c3", "c1": "c1",
            "c0": "c0"}[wl]
    cfg = gen.get_config(base, top_p=args.top_p) if args.top_p else gen.get_config(base)
    dtype = {"c4i2": gen.I2, "c2i8": gen.I8}.get(wl, cfg.expert_dtype)
    T = (args.batch if base == "c4" else None) or (16 if base == "c4" else cfg.batches[0])
    L = args.layers if base in ("c2", "c3", "c4") else 1
    if base == "c3":
        L = min(L, 2)
    if dtype == gen.I8:
        L = min(L, 4)   # 4 int8 layers hold as many bytes as 8 int4 ones (~39 GB)

    # ---- inputs, resident in HBM before timing
    if base in ("c0", "c1"):
        layers = [gdev.upload_host_layer(gen.host_layer(cfg, l, experts="all"), dev)
                  for l in range(L)]
    else:
        layers = [gdev.generate_device_layer(cfg, l, dev, dtype=dtype) for l in range(L)]
    P = 64 if T <= 16 else 2
    xs = []
    for p in range(P):
        x = gen.x_tokens(cfg, T, batch_id=1000 + p)
        xs.append(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev))
    desc = capi.make_desc(layers[0].desc_spec)
    weights = [capi.make_weights(l.pointers()) for l in layers]
    nb = capi.moe_workspace_bytes(desc, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # ---- unique experts per step (library routing, computed before timing)
    n_active = []
    kept_slots = []
    for i in range(max(K, 1)):
        l, p = i % L, i % P
        if i < P * L:
            capi.moe_route(desc, layers[l].w_router, layers[l].bias, xs[p], T, idx, tw, ws, nb)
            ih = idx.cpu().numpy()
            n_active.append(len(np.unique(ih[ih >= 0])))
            kept_slots.append(int((ih >= 0).sum()))
        else:
            n_active.append(n_active[i % (P * L)])

    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    stage_ids = list(range(capi.MOE_N_STAGES)) if args.stages else [capi.MOE_STAGE_GATE_UP]
    evs = [[[hip.event(), hip.event()] for _ in stage_ids] for _ in range(K)]
    # an empty event pair per step: what an event bracket adds by itself
    evp = [[hip.event(), hip.event()] for _ in range(K)]
    # an event pair around each whole step (a replay of its own)
    evw = [[hip.event(), hip.event()] for _ in range(K)]

    def step(i, timed, whole=False):
        l, p = i % L, i % P
        events = None
        cap = not args.eager
        if timed:
            events = [0] * (2 * capi.MOE_N_STAGES)
            for k, s_id in enumerate(stage_ids):
                events[2 * s_id], events[2 * s_id + 1] = evs[i][k]
            hip.record(evp[i][0], sh, cap)
            hip.record(evp[i][1], sh, cap)
        if whole:
            hip.record(evw[i][0], sh, cap)
        capi.moe_layer_forward_ex(desc, weights[l], xs[p], T, out, None, None, ws, nb,
                                  stream=sh, events=events)
        if whole:
            hip.record(evw[i][1], sh, cap)

    rep_ms = []
    ab = None
    # The headline loop carries no event nodes; per-kernel durations come from a
    # second pass over the same K steps with events around the stages.
    if args.eager:
        for i in range(W):
            step(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i, False)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(K):
            step(i, True)
        torch.cuda.synchronize()
        for i in range(K):
            step(i, False, whole=True)
        torch.cuda.synchronize()
    else:
        step(0, False)                       # first launches outside any capture
        torch.cuda.synchronize()
        gw = hip.capture(sh, lambda: [step(i, False) for i in range(W)])
        gt = hip.capture(sh, lambda: [step(i, False) for i in range(K)])
        ge = hip.capture(sh, lambda: [step(i, True) for i in range(K)])
        gb = hip.capture(sh, lambda: [step(i, False, whole=True) for i in range(K)])
        hip.launch(gw, sh)
        # the timed graph is uploaded before the timed region (its first
        # launch would otherwise carry the upload of its 3K nodes)
        hip.upload(gt, sh)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hip.launch(gt, sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        hip.launch(ge, sh)
        torch.cuda.synchronize()
        hip.launch(gb, sh)
        torch.cuda.synchronize()
        # further replays of the same K steps: the spread of the step time
        r0, r1 = hip.event(), hip.event()
        for _ in range(replays):
            hip.record(r0, sh, False)
            hip.launch(gt, sh)
            hip.record(r1, sh, False)
            torch.cuda.synchronize()
            rep_ms.append(hip.elapsed_ms(r0, r1) / K)
        if ab_lib:
            ab = ab_compare(hip, capi, ab_lib, gt, sh, out, lambda: [step(i, False) for i in range(K)],
                            K, replays)

    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / K
    value = K * T / elapsed
    stage_ms = {}
    for k, s_id in enumerate(stage_ids):
        stage_ms[s_id] = [hip.elapsed_ms(evs[i][k][0], evs[i][k][1]) for i in range(K)]
    # The event bracket holds the kernel plus what the two event nodes add
    # around running work.  That is measured on whole steps: a bracket around
    # each step of a replay of its own, less the event-free time per step
    # (the median over the event-timed replays of the step graph; the host
    # clock's step time when there are none).  An empty event pair, also
    # printed, takes longer than the nodes add around a kernel.  Medians over
    # the steps, as a few brackets now and then take several times their
    # usual time.
    bracket_ms = float(np.median(stage_ms[capi.MOE_STAGE_GATE_UP]))
    pair_ms = float(np.median([hip.elapsed_ms(a, b) for a, b in evp]))
    whole = [hip.elapsed_ms(a, b) for a, b in evw]
    whole_ms = float(np.median(whole))
    free_ms = float(np.median(rep_ms)) if rep_ms else ms_step
    over_ms = whole_ms - free_ms
    gu_ms = bracket_ms - over_ms if 0.0 < over_ms < 0.5 * bracket_ms else bracket_ms
    gu_bytes = float(np.mean([gate_up_bytes(cfg, dtype, n, T) for n in n_active[:K]]))
    lay_bytes = float(np.mean([layer_bytes(cfg, dtype, n, T) for n in n_active[:K]]))
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9

    if base == "c3":
        # prefill: the grouped GEMM on the matrix cores, priced in flops
        flops = gate_up_flops(cfg, T)
        tflops = flops / (gu_ms * 1e-3) / 1e12
        roofline = {
            "kernel": ("gate/up stage: moe::k_ggemm int4 routed tiles + the bf16 shared expert"
                       " (hipBLASLt GEMM + moe::k_swiglu_rows at >= 256 tokens)"),
            "bound": "mfma",
            "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": int(flops),
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "bracket_us": round(bracket_ms * 1e3, 3),
            "event_pair_us": round(pair_ms * 1e3, 3),
            "bracket_overhead_us": round(over_ms * 1e3, 3),
        }
    else:
        sel = T == 1 and shared_runs_with_router(cfg, dtype, T)
        roofline = {
            "kernel": ("moe::k_gemv_sel routed gate/up + SwiGLU (the selection and the shared"
                       " expert's down projection in the same launch)"
                       if sel and shared_down_in_gate_up(cfg, dtype, T) else
                       "moe::k_gemv_sel routed gate/up + SwiGLU (the selection in the same launch)"
                       if sel else
                       "moe::k_gemv gate/up + SwiGLU (routed experts)"
                       if shared_runs_with_router(cfg, dtype, T) else
                       "moe::k_gemv gate/up + SwiGLU (routed and shared experts)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            # counters were taken on the default workload (one token, all 8 experts)
            "traffic": measured_traffic(wl) if (T == 1 and not cfg.top_p) else None,
            "bytes_per_launch": int(gu_bytes),
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "bracket_us": round(bracket_ms * 1e3, 3),
            "event_pair_us": round(pair_ms * 1e3, 3),
            "bracket_overhead_us": round(over_ms * 1e3, 3),
        }
    names = {capi.MOE_STAGE_ROUTE: "route", capi.MOE_STAGE_BUCKET: "bucket",
             capi.MOE_STAGE_GATE_UP: "gate_up", capi.MOE_STAGE_DOWN: "down",
             capi.MOE_STAGE_COMBINE: "combine"}
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.act_dtype == gen.F32 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: H={cfg.hidden} I={cfg.inter} E={cfg.n_experts} "
                        f"top-{cfg.top_k} ({'softmax' if cfg.router else 'sigmoid noaux_tc'}) "
                        f"{ {gen.I4: 'int4', gen.I2: 'int2', gen.I8: 'int8', gen.BF16: 'bf16'}[dtype]} experts, "
                        f"{T} token(s)/step, {L} rotating layer instance(s)"
                        + (f", adaptive expert top-p {cfg.top_p}" if cfg.top_p else ""),
            "global_batch": T,
            "seq_len": 1,
            "parallelism": "single_gpu",
            "launch": "eager" if args.eager else "hip_graph",
        },
        "layer_hbm_gbps": round(lay_bytes / (ms_step * 1e-3) / 1e9, 1),
        "layer_bytes_per_step": int(lay_bytes),
        "routing": {"top_p": cfg.top_p,
                    "experts_per_token": round(float(np.mean(kept_slots)) / T, 3),
                    "unique_experts_per_step": round(float(np.mean(n_active[:K])), 2)},
        "roofline": roofline,
    }
    # per-step time: over further replays of the K steps (each replay's mean),
    # and over the steps of the bracketed replay (each step's bracket)
    if rep_ms:
        res["step_us"] = dict(replays=len(rep_ms), **percentiles(np.array(rep_ms) * 1e3))
        res["step_us"]["per_step_bracket"] = percentiles(np.array(whole) * 1e3)
    if args.stages:
        res["stage_us"] = {names[s_id]: round(1e3 * float(np.mean(v)), 3)
                           for s_id, v in stage_ms.items()}
    if ab is not None:
        res["ab"] = ab
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, dtype, T, args.cpu_seconds)
    del layers, ws, xs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def ab_compare(hip, capi, lib_b, graph_a, sh, out, capture_steps, K, pairs):
    """ABBA comparison of the in-tree library (A) with another build of it (B,
    the path given): B's steps are captured with B's library, the two graphs are
    replayed in the order A B B A, `pairs` times, and the per-step times
    compared.  Gated on the outputs: the last step's output after a replay of
    A and of B must be the same bits (a variant that changes the result is not
    an A/B of the same computation)."""
    import hashlib
    import torch
    lib_a = capi.lib()
    capi._lib = capi.load_library(lib_b)
    try:
        # one eager pass first, as the in-tree library had before its capture:
        # set-up that a library does only outside capture (a GEMM library handle
        # and its plans) is then in place for B's graph too
        capture_steps()
        torch.cuda.synchronize()
        graph_b = hip.capture(sh, capture_steps)
    finally:
        capi._lib = lib_a
    r0, r1 = hip.event(), hip.event()

    def replay(g):
        hip.record(r0, sh, False)
        hip.launch(g, sh)
        hip.record(r1, sh, False)
        torch.cuda.synchronize()
        return hip.elapsed_ms(r0, r1) / K, hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest()

    ta, tb, ha, hb = [], [], set(), set()
    for _ in range(pairs):
        for g, t, h in ((graph_a, ta, ha), (graph_b, tb, hb), (graph_b, tb, hb), (graph_a, ta, ha)):
            ms, digest = replay(g)
            t.append(ms)
            h.add(digest)
    ma, mb = float(np.median(ta)), float(np.median(tb))
    return {"lib_b": lib_b, "order": "ABBA", "pairs": pairs,
            "a_us": percentiles(np.array(ta) * 1e3), "b_us": percentiles(np.array(tb) * 1e3),
            "b_over_a": round(mb / ma, 4), "outputs_identical": ha == hb and len(ha) == 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="c2",
                    choices=["c2", "c2i8", "c4i4", "c4i2", "c3", "c1", "c0", "requant"])
    ap.add_argument("--batch", type=int, default=None, help="tokens per step (c4: 2, 4 or 16)")
    ap.add_argument("--layers", type=int, default=8, help="distinct layer instances rotated")
    ap.add_argument("--eager", action="store_true", help="launch each step eagerly (no graph)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill (c3) measurement the default workload also reports")
    ap.add_argument("--replays", type=int, default=5,
                    help="further replays of the timed steps for the spread of the step time")
    ap.add_argument("--ab", default=None, metavar="LIBMOE_SO",
                    help="also time another build of libmoe.so against the in-tree one, "
                         "ABBA-interleaved, gated on identical outputs")
    ap.add_argument("--stages", action="store_true", help="also time every stage")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="adaptive expert top-p (0: off): the router keeps the shortest prefix "
                         "of each token's top-k whose routing mass reaches this share")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy five times (the known-size kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return

    if args.workload == "requant":
        return bench_requant(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU sharding is a design "
                                   "only (expert-parallel by router group), --gpus must be 1"}))
        sys.exit(2)

    res = run_workload(args, args.workload, args.steps, args.warmup, not args.no_cpu_baseline,
                       replays=args.replays, ab_lib=args.ab)
    if args.workload == "c2" and not args.no_prefill and not args.top_p:
        # the prefill workload on the same box, GPU only: the grouped GEMM on
        # the matrix cores
        pf_args = argparse.Namespace(**{**vars(args), "stages": False})
        pf = run_workload(pf_args, "c3", 20, 5, False, replays=args.replays)
        res["prefill"] = {
            "workload": pf["config"]["workload"],
            "steps": pf["steps"],
            "ms_per_step": pf["ms_per_step"],
            "tokens_per_s": pf["value"],
            "step_us": pf.get("step_us"),
            "gate_up_tflops": pf["roofline"]["achieved"],
            "gate_up_mfma_frac": pf["roofline"]["frac"],
            "gate_up_us": pf["roofline"]["avg_launch_us"],
            "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
