#!/usr/bin/env python3
"""Throughput of the folded multi-branch verify layer on one MI355X.

A step is one complete verify layer (gate, provenance, packing, packed QKV GEMM, prefix
and block attention with per-branch correction, O projection, packed SwiGLU FFN,
combine) over the parent and all draft branches of one synthetic block, with every
input already resident in HBM.  The default workload is the 7B-shaped layer (hidden
3584, 28/4 heads x 128, FFN 18944, prefix 512, block 32, a 3-ary draft tree of
1 + 15 nodes, tau = 0.05).  `value` is branch-tokens verified per second per layer
(N*B slots per step); `us_per_verify_layer` is the same number as latency.

The default run also reports, in the same JSON line: per-step p10/p50/p90, per-kernel
times and roofline fractions, selection cost (gate + provenance/packing) and correction
cost (against the REUSE variant), the tau sweep of the 3B-shaped DAG layer (recompute
fraction against time), the 28-layer 7B-shaped stack's step time, on-box measured HBM
copy and bf16 GEMM rates beside the published peaks, and the CPU oracle's rate at all
host cores and at one BLAS thread.

Prints exactly one JSON line on stdout; progress goes to stderr.  --report PATH writes
the extended results (per-kernel times per tau, per-step samples) as JSON."""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, public spec
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "dominant_kernel_traffic.json")
COPY_BYTES = 256 << 20         # calibration copy: bytes read (and written) per launch
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, public spec
FP32_PEAK_TFLOPS = 157.3       # dense fp32


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t helpers from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.h.hipEventRecord(ev, stream) == 0

    def ms(self, a, b):
        """Elapsed ms between two recorded events (None if the pair was never recorded)."""
        assert self.h.hipEventSynchronize(b) == 0
        v = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            self.h.hipGetLastError()          # clear: the pair was never recorded
            return None
        return v.value

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def algorithmic(cfg, K):
    """Bytes and flops each kernel must move/compute per launch (weights read once, packed
    rows only, prefix read once per KV head)."""
    eb = 2 if cfg.dtype == "bf16" else 4
    d, ff, dh, nq, nkv, S, P, B = (cfg.hidden, cfg.ffn, cfg.head_dim, cfg.n_q, cfg.n_kv,
                                   cfg.slots, cfg.prefix, cfg.block)
    qkvd = cfg.qkv_dim
    g = nq // nkv
    out = {
        "gate": dict(bytes=2 * S * d * eb + S * 9, flops=4 * S * d),
        "resolve_pack": dict(bytes=S * 1 + cfg.num_nodes * 4 + 3 * S * 4 + 4, flops=0),
        "qkv": dict(bytes=qkvd * d * eb + K * d * eb + K * qkvd * eb, flops=2 * K * d * qkvd),
        "attn_prefix": dict(bytes=2 * P * nkv * dh * eb + K * nq * dh * eb,
                            flops=4 * K * nq * P * dh),
        "attn_block": dict(bytes=K * qkvd * eb + S * nq * dh * eb, flops=4 * S * nq * B * dh),
        # O projection and its finish (residual add, FFN RMSNorm of the packed rows)
        "o_proj+o_finish": dict(bytes=d * nq * dh * eb + S * nq * dh * eb + 2 * S * d * eb
                                + K * d * eb, flops=2 * S * nq * dh * d),
        "ffn_gate_up": dict(bytes=2 * ff * d * eb + K * d * eb + K * ff * eb,
                            flops=2 * K * d * 2 * ff),
        "ffn_down": dict(bytes=d * ff * eb + K * ff * eb + K * d * eb, flops=2 * K * ff * d),
        "combine": dict(bytes=2 * S * d * eb + K * d * eb, flops=S * d),
    }
    return out


def kernel_rooflines(cfg, K, kernels):
    """Per-kernel achieved HBM rate and MFMA rate from the probe times and the
    algorithmic bytes/flops, as fractions of MI355X peak."""
    alg = algorithmic(cfg, K)
    times = dict(kernels)
    if "o_proj" in times and "o_finish" in times:
        times["o_proj+o_finish"] = times["o_proj"] + times["o_finish"]
    peak_tf = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    out = {}
    for name, a in alg.items():
        us = times.get(name)
        if not us:
            continue
        gbs = a["bytes"] / (us * 1e-6) / 1e9
        tfs = a["flops"] / (us * 1e-6) / 1e12
        out[name] = dict(us=us, GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS, TFLOPs=tfs,
                         mfma_frac=tfs / peak_tf, bytes=a["bytes"], flops=a["flops"])
    return out


# Copies of one layer's weights that successive calls take in turn.  In a model each layer's
# weights are read once per verify step, with every other layer's weights streamed in
# between, so none of them is still in the GPU's 256 MB memory-side cache when the layer comes
# round again.  Timing one layer over and over with one set of weights would let the weights
# that the FFN stream leaves in that cache (QKV, O and down, ~195 MB at the 7B shape) be hit on
# the next call: 15 us per 7B layer faster than the model would run.  Three copies (1.4 GB at
# the 7B shape) cycle through more than the cache holds.
WEIGHT_COPIES = 3


def build_layer(cfg, copies=WEIGHT_COPIES):
    import numpy as np  # noqa: F401
    from branch_folding_amd.runner import DeviceLayer
    from synth import make_workload
    t = time.time()
    w = make_workload(cfg, layers=1)
    log(f"[bench] workload {cfg.name} drawn in {time.time() - t:.1f}s")
    dl = rotating(DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src), copies)
    return w, dl


def rotating(dl, copies=WEIGHT_COPIES):
    """Makes successive dl.forward calls take the layer's weights from `copies` copies in
    turn (the first is dl's own)."""
    if copies > 1:
        sets = [dl.w] + [{k: v.clone() for k, v in dl.w.items()} for _ in range(copies - 1)]
        base, turn = dl.forward, [0]

        def forward(*a, **k):
            dl.w = sets[turn[0] % len(sets)]
            turn[0] += 1
            return base(*a, **k)
        dl.forward = forward
    return dl


def time_layer(dl, tau, steps, warmup, ev, stream, probe_step=None):
    """Returns (ms per step, list of probe-step durations in ms)."""
    import torch
    from branch_folding_amd import _lib as L
    for _ in range(warmup):
        dl.forward(tau, stream=stream)
    t0, t1 = ev.create(2)
    ps = ev.create(steps) if probe_step is not None else []
    pe = ev.create(steps) if probe_step is not None else []
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for i in range(steps):
        probe = None
        if probe_step is not None:
            probe = L.Probe(probe_step, ps[i], pe[i])
        dl.forward(tau, stream=stream, probe=probe)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    total = ev.ms(t0, t1)
    per = [x for x in (ev.ms(a, b) for a, b in zip(ps, pe)) if x is not None]
    ev.destroy([t0, t1] + ps + pe)
    return total / steps, per


def time_reuse(dl, tau, steps, warmup, ev, stream):
    """ms per step of the layer with the REUSE attention variant."""
    import torch
    for _ in range(warmup):
        dl.forward(tau, stream=stream, reuse=True)
    t0, t1 = ev.create(2)
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(steps):
        dl.forward(tau, stream=stream, reuse=True)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    ev.destroy([t0, t1])
    return ms


def kernel_breakdown(dl, tau, reps, ev, stream):
    from branch_folding_amd import _lib as L
    out = {}
    for idx, name in enumerate(L.STEPS):
        _, per = time_layer(dl, tau, reps, 2, ev, stream, probe_step=idx)
        if per:                      # steps fused into another launch record nothing
            out[name] = sum(per) / len(per) * 1e3
    return out


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` at `workload` from the committed rocprofv3 counter
    record, or None when there is no record for that kernel and workload or the kernel's
    source has changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("workload") != workload:
        return None
    # every source file of the kernel's translation unit, hashed in the listed order
    h = hashlib.sha256()
    try:
        for src in rec.get("sources", []):
            h.update(open(os.path.join(ROOT, src), "rb").read())
    except OSError:
        return None
    ok = rec.get("sources") and h.hexdigest() == rec.get("sources_sha256")
    return rec.get("hbm_bytes_per_launch") if ok else None


def calibration_copy(reps=3):
    """A plain device-to-device copy of known size; its FETCH_SIZE / WRITE_SIZE readings
    scale the counters of the other kernels to bytes."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def _oracle_rate(w, tau, budget_s):
    from oracle import layer
    cfg = w.cfg
    pk, pv = w.prefix_kv(0)
    runs, t0 = 0, time.time()
    while True:
        layer(w.weights[0], w.H, w.fold_src, tau, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
              eps=cfg.rms_eps)
        runs += 1
        el = time.time() - t0
        if el >= budget_s:
            break
    return cfg.slots * runs / el, runs, el


def cpu_baseline(w, tau, budget_s):
    """The oracle as it stands on the host cores, on whole verify layers of the same
    workload, repeated until the time budget is used: once with the BLAS pool at every
    core it starts with, once limited to one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    v, runs, el = _oracle_rate(w, tau, budget_s)
    with threadpool_limits(limits=1):
        v1, runs1, el1 = _oracle_rate(w, tau, budget_s)
    cfg = w.cfg
    return dict(value=v, unit="branch-tokens/s", cores=int(cores), kind="oracle",
                sample=f"{runs} whole {cfg.name} verify layers (tau={tau}), numpy float64 "
                       f"oracle, {el:.1f}s wall at {cores} BLAS threads; "
                       f"{os.cpu_count()} host CPUs visible",
                value_1_thread=v1,
                sample_1_thread=f"{runs1} whole layers, {el1:.1f}s wall at 1 BLAS thread")


def step_distribution(dl, tau, steps, ev, stream):
    """Per-step durations (us) from a separate pass with an event pair around every step
    (the timed pass that gives `value` carries no events inside)."""
    import torch
    evs = ev.create(2 * steps)
    torch.cuda.synchronize()
    for i in range(steps):
        ev.record(evs[2 * i], stream)
        dl.forward(tau, stream=stream)
        ev.record(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    per = sorted(ev.ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(steps))
    ev.destroy(evs)

    def q(f):
        return per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    return dict(p10=q(0.1), p50=q(0.5), p90=q(0.9), min=per[0], max=per[-1], n=len(per))


def vendor_gemm(cfg, K, ev, stream):
    """The same four products as the layer's GEMMs, through torch.matmul (hipBLASLt), each
    timed alone: QKV and the FFN on the K packed rows, the O projection on all S slots.
    Plain products only (no gather, SwiGLU, residual or split reduction); three weight
    copies in turn, so that, as in the layer, the weights come from HBM and not from the
    memory-side cache.  A reference point for the layer's kernels, not part of the step."""
    import torch
    d, ff, qd, S = cfg.hidden, cfg.ffn, cfg.n_q * cfg.head_dim, cfg.slots
    shapes = {"qkv": (K, d, cfg.qkv_dim), "o_proj": (S, qd, d),
              "ffn_gate_up": (K, d, 2 * ff), "ffn_down": (K, ff, d)}
    out = {}
    for name, (m, k, n) in shapes.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        ws = [torch.randn(n, k, device="cuda", dtype=torch.bfloat16) for _ in range(3)]
        c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
        for i in range(6):
            torch.matmul(a, ws[i % 3].t(), out=c)
        t0, t1 = ev.create(2)
        torch.cuda.synchronize()
        ev.record(t0, stream)
        reps = 30
        for i in range(reps):
            torch.matmul(a, ws[i % 3].t(), out=c)
        ev.record(t1, stream)
        torch.cuda.synchronize()
        out[name] = ev.ms(t0, t1) * 1e3 / reps
        ev.destroy([t0, t1])
        del a, ws, c
    torch.cuda.empty_cache()
    return out


def measured_peaks(ev, stream):
    """On-box reference rates beside the published peaks: a 1 GiB device-to-device copy
    (bytes read + written per second) and an 8192^3 bf16 GEMM through torch (hipBLASLt)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    x = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    out = {}
    for name, fn, work in (("hbm_copy_GBps", lambda: b.copy_(a), 2 * n / 1e9),
                           ("bf16_gemm_TFLOPs", lambda: torch.mm(x, y), 2 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        t0, t1 = ev.create(2)
        torch.cuda.synchronize()
        ev.record(t0, stream)
        reps = 10
        for _ in range(reps):
            fn()
        ev.record(t1, stream)
        torch.cuda.synchronize()
        out[name] = work * reps / (ev.ms(t0, t1) * 1e-3)
        ev.destroy([t0, t1])
    del a, b, x, y
    torch.cuda.empty_cache()
    out["hbm_copy_frac_of_peak"] = out["hbm_copy_GBps"] / HBM_PEAK_GBS
    out["bf16_gemm_frac_of_peak"] = out["bf16_gemm_TFLOPs"] / BF16_PEAK_TFLOPS
    return out


# probe steps that are a single kernel (or a GEMM and its own split-K reduction) with an
# algorithmic byte / flop count: candidates for the roofline of the dominant kernel
ROOFLINE_STEPS = ("gate", "resolve_pack", "qkv", "attn_prefix", "attn_block", "ffn_gate_up",
                  "ffn_down", "combine")


def roofline_of(cfg, K, name, us, workload):
    """Roofline object of one kernel: HBM-bound if its algorithmic arithmetic intensity is
    below the ridge point of its dtype, else MFMA-bound."""
    a = algorithmic(cfg, K)[name]
    peak_tf = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = a["flops"] / max(a["bytes"], 1)
    if ai < ridge:
        achieved = a["bytes"] / (us * 1e-6) / 1e9
        out = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                   frac=achieved / HBM_PEAK_GBS)
    else:
        achieved = a["flops"] / (us * 1e-6) / 1e12
        out = dict(bound="mfma", achieved=achieved, peak=peak_tf, unit="TFLOP/s",
                   frac=achieved / peak_tf)
    out.update(traffic=measured_traffic(name, workload), kernel=name, avg_us=us,
               algorithmic_bytes=a["bytes"], algorithmic_flops=a["flops"],
               arithmetic_intensity=ai, ridge=ridge)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4],
                    help="configuration id (1 = the 7B-shaped headline layer; 3 times one "
                         "layer of the 28-layer stack's shape)")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget per thread setting (all cores, then one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the tau sweep of the 3B-shaped DAG layer")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 28-layer stack's end-to-end step time")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the on-box copy and GEMM reference rates")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip timing the REUSE variant (the correction cost)")
    ap.add_argument("--only-layer", action="store_true",
                    help="time the selected layer only: no sweep, stack, reference rates, "
                         "REUSE variant or CPU baseline (for profiler runs)")
    ap.add_argument("--budget-sweep", action="store_true",
                    help="also run the draft-budget sweep: the 7B layer at 1+{3,7,15,31,63} "
                         "branches, dense and folded")
    ap.add_argument("--gate-sweep", action="store_true",
                    help="also time specfold_gate alone on hidden states of 34 to 134 MB")
    ap.add_argument("--rope-bias", action="store_true",
                    help="also time the layer with the rotary embedding (base 10^6) and QKV "
                         "bias of the 7B model family")
    ap.add_argument("--lm-head", action="store_true",
                    help="also time the LM head + per-branch argmax (vocab 152064) on the 7B "
                         "layer's packed rows")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--report", default=None)
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel probes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help=f"also run a {COPY_BYTES >> 20} MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.only_layer:
        args.no_sweep = args.no_stack = args.no_peaks = args.no_reuse = True
        args.no_cpu_baseline = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the folded verify layer is measured on one "
              "MI355X (multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from branch_folding_amd import _lib as L
    from synth import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.lib()
    cfg = CONFIGS[args.workload]
    tau = cfg.tau if args.tau is None else args.tau
    w, dl = build_layer(cfg)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()

    dl.forward(tau, stream=stream)
    torch.cuda.synchronize()
    K = dl.fold_state()["K"]
    log(f"[bench] K={K} of S={cfg.slots} packed rows")

    # the timed steps carry no probe events
    ms, _ = time_layer(dl, tau, args.steps, args.warmup, ev, stream)
    log(f"[bench] {ms * 1e3:.1f} us per verify layer")
    dist = step_distribution(dl, tau, args.steps, ev, stream)
    log(f"[bench] per step p10/p50/p90 {dist['p10']:.1f} / {dist['p50']:.1f} / "
        f"{dist['p90']:.1f} us (event pair around every step)")
    kernels = {} if args.no_breakdown else kernel_breakdown(dl, tau, 20, ev, stream)
    if kernels:
        log("[bench] per-kernel us: " + ", ".join(f"{k}={v:.1f}" for k, v in kernels.items()))
    # the dominant kernel (the longest single-kernel step) is timed again in a pass of the
    # same length with events around its launch only
    cand = {k: v for k, v in kernels.items() if k in ROOFLINE_STEPS}
    dom_name = max(cand, key=cand.get) if cand else "ffn_gate_up"
    _, per = time_layer(dl, tau, args.steps, 2, ev, stream, probe_step=L.STEPS.index(dom_name))
    dom_us = sum(per) / len(per) * 1e3
    roof = roofline_of(cfg, K, dom_name, dom_us, cfg.name)
    log(f"[bench] dominant kernel {dom_name}: {dom_us:.1f} us, {roof['achieved']:.0f} "
        f"{roof['unit']} ({roof['frac'] * 100:.1f}% of the {roof['bound']} peak)")
    if args.calibrate_copy:
        calibration_copy()
    ms_r = None if args.no_reuse else time_reuse(dl, tau, args.steps, args.warmup, ev, stream)
    if ms_r is not None:
        log(f"[bench] REUSE variant {ms_r * 1e3:.1f} us per verify layer")

    unit_metric = ("branch-tokens verified/s per layer "
                   f"({cfg.name}: hidden {cfg.hidden}, {cfg.num_nodes} nodes x block "
                   f"{cfg.block}, prefix {cfg.prefix}, tau {tau}); us/verify-layer")
    result = {
        "metric": unit_metric,
        "value": cfg.slots / (ms * 1e-3),
        "unit": "branch-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; random-init weights of the named shape)",
        "config": {"workload": cfg.name, "nodes": cfg.num_nodes, "block": cfg.block,
                   "hidden": cfg.hidden, "heads": f"{cfg.n_q}q/{cfg.n_kv}kv x {cfg.head_dim}",
                   "ffn": cfg.ffn, "prefix": cfg.prefix, "tau": tau, "graph": cfg.graph,
                   "weight_copies": WEIGHT_COPIES},
        "us_per_verify_layer": ms * 1e3,
        "us_per_step_dist": dist,
        "packed_rows": K,
        "recompute_fraction": K / cfg.slots,
        "kernels_us": kernels,
        "kernels_roofline": kernel_rooflines(cfg, K, kernels) if kernels else {},
        "selection_us": (kernels.get("gate", 0.0) + kernels.get("resolve_pack", 0.0)
                         if kernels else None),
        "reuse": (None if ms_r is None else
                  dict(us_per_verify_layer=ms_r * 1e3, correction_cost_us=(ms - ms_r) * 1e3)),
        "roofline": roof,
    }
    report = {"main": result}
    if not args.no_peaks:
        result["measured_peaks"] = measured_peaks(ev, stream)
        log("[bench] on-box reference rates: " + ", ".join(
            f"{k}={v:.3g}" for k, v in result["measured_peaks"].items()))
        if cfg.dtype == "bf16" and K > 0:
            result["vendor_gemm_us"] = vendor_gemm(cfg, K, ev, stream)
            log("[bench] the same GEMM shapes through torch.matmul (hipBLASLt), us: " + ", ".join(
                f"{k}={v:.1f}" for k, v in result["vendor_gemm_us"].items()))
    if args.gate_sweep:
        report["gate_sweep"] = gate_sweep(ev, stream)
        result["gate_sweep"] = report["gate_sweep"]
    if args.rope_bias:
        crb = cfg.with_(name=cfg.name + "-rope-bias", rope_theta=1.0e6, qkv_bias=True)
        _, dlr = build_layer(crb)
        ms_rb, _ = time_layer(dlr, tau, args.steps, args.warmup, ev, stream)
        result["rope_bias"] = dict(us_per_verify_layer=ms_rb * 1e3,
                                   extra_us=(ms_rb - ms) * 1e3)
        log(f"[bench] with rotary embedding + QKV bias: {ms_rb * 1e3:.1f} us per verify layer "
            f"({(ms_rb - ms) * 1e3:+.1f} us)")
        del dlr
        torch.cuda.empty_cache()
    if args.lm_head:
        report["lm_head"] = lm_head_bench(cfg, w, dl, tau, ev, stream, args.steps, args.warmup)
        result["lm_head"] = report["lm_head"]
    del dl
    torch.cuda.empty_cache()
    if args.budget_sweep:
        report["budget_sweep"] = budget_sweep(w, ev, stream, args.steps, args.warmup)
        result["budget_sweep"] = [{k: r[k] for k in ("branches", "tau", "K", "us",
                                                     "branch_tokens_per_s")}
                                  for r in report["budget_sweep"]]
    if not args.no_sweep:
        report["tau_sweep"] = tau_sweep(ev, stream, args.steps, args.warmup)
        result["tau_sweep"] = {"workload": CONFIGS[2].name,
                               "rows": [{k: r[k] for k in ("tau", "K", "recompute_fraction",
                                                           "us", "speedup_vs_dense")}
                                        for r in report["tau_sweep"]]}
    if not args.no_stack:
        report["stack"] = stack_bench(ev, stream, args.stack_steps, 3)
        result["stack"] = {k: report["stack"][k] for k in
                           ("workload", "layers", "us_per_verify_step", "us_per_layer",
                            "us_per_verify_step_graph", "packed_rows_per_layer", "weights")}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (all BLAS threads, then one) ...")
        result["cpu_baseline"] = cpu_baseline(w, tau, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    if args.report:
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(result), flush=True)


def tau_sweep(ev, stream, steps, warmup):
    """Recompute fraction and time of the 3B-shaped DAG layer across tau (dense first)."""
    import torch
    from synth import CONFIGS
    cfg = CONFIGS[2]
    w, dl = build_layer(cfg)
    rows = []
    for tau in (-1.0,) + tuple(cfg.taus):
        dl.forward(tau, stream=stream)
        torch.cuda.synchronize()
        K = dl.fold_state()["K"]
        ms, _ = time_layer(dl, tau, steps, warmup, ev, stream)
        kern = kernel_breakdown(dl, tau, 10, ev, stream)
        rows.append(dict(tau=tau, K=K, recompute_fraction=K / cfg.slots, us=ms * 1e3,
                         speedup_vs_dense=rows[0]["us"] / (ms * 1e3) if rows else 1.0,
                         kernels_us=kern))
        log(f"[bench] sweep tau={tau}: K={K} ({K / cfg.slots:.3f}) {ms * 1e3:.1f} us")
    del dl
    torch.cuda.empty_cache()
    return rows


def lm_head_bench(cfg, w, dl, tau, ev, stream, steps, warmup):
    """The step after the last layer: logits of the packed rows against a [152064, d] LM
    head and every branch's argmax token, with the fold state the layer just produced
    (specfold_lm_head_argmax).  Algorithmic bytes: the head once, the packed rows, the
    hidden states' normalisation pass and the token outputs."""
    import torch
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import shape_of
    from synth import VOCAB_7B, lm_head_weights
    g, wl = lm_head_weights(cfg, VOCAB_7B)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gd = torch.from_numpy(g).to(dt).cuda()
    wd = torch.from_numpy(wl).to(dt).cuda()
    del wl
    dl.forward(tau, stream=stream)
    torch.cuda.synchronize()
    st = dl.state                      # the layer's fold state, on the device
    hid = dl.out                       # the layer's output stands in for the final hidden states
    sh = shape_of(cfg)
    S, K, d = cfg.slots, dl.fold_state()["K"], cfg.hidden
    nb = L.specfold_lm_head_workspace_bytes(sh, VOCAB_7B)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    rt = torch.empty(S, dtype=torch.int32, device="cuda")
    rl = torch.empty(S, dtype=torch.float32, device="cuda")
    tok = torch.empty(S, dtype=torch.int32, device="cuda")
    call = lambda: L.specfold_lm_head_argmax(sh, VOCAB_7B, gd, wd, hid, st["packed_slot"],
                                             st["slot_row"], st["packed_count"], rt, rl, tok,
                                             ws, nb, stream)
    for _ in range(warmup):
        call()
    t0, t1 = ev.create(2)
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(steps):
        call()
    ev.record(t1, stream)
    torch.cuda.synchronize()
    us = ev.ms(t0, t1) / steps * 1e3
    ev.destroy([t0, t1])
    eb = 2 if cfg.dtype == "bf16" else 4
    alg = VOCAB_7B * d * eb + S * d * eb * 2 + K * d * eb + S * 4
    res = dict(vocab=VOCAB_7B, packed_rows=K, us=us, GBps=alg / (us * 1e-6) / 1e9,
               hbm_frac=alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, algorithmic_bytes=alg)
    log(f"[bench] LM head (vocab {VOCAB_7B}, {K} packed rows, {S} slots): {us:.1f} us, "
        f"{res['GBps']:.0f} GB/s ({res['hbm_frac'] * 100:.0f}% of HBM peak)")
    del wd, ws
    torch.cuda.empty_cache()
    return res


def gate_sweep(ev, stream, reps=50):
    """Streaming rate of the gate kernel alone (specfold_gate: ratios and masks) at the
    stress layer's row shape (hidden 4096, block 64, bf16, 3-ary tree) with 64 to 256
    nodes, i.e. 33.6 MB to 134 MB of hidden states (256 x 64 is the largest slot count
    one call takes).  Algorithmic bytes count every row
    once (a parent row is also some other branch's own row) plus the 5 output bytes per
    slot; the rate is also given against the child + parent reads the kernel issues."""
    import torch
    from branch_folding_amd import _lib as L
    d, B = 4096, 64
    rows = []
    for n in (64, 128, 256):
        S = n * B
        g = torch.Generator(device="cuda").manual_seed(n)
        H = torch.randn(S * d, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
        fs = torch.tensor([-1] + [(m - 1) // 3 for m in range(1, n)], dtype=torch.int32,
                          device="cuda")
        ratio = torch.empty(S, dtype=torch.float32, device="cuda")
        rec = torch.empty(S, dtype=torch.uint8, device="cuda")
        sh = L.Shape(num_nodes=n, block=B, hidden=d, n_q_heads=32, n_kv_heads=4, head_dim=128,
                     ffn=14336, prefix_len=0, rms_eps=1e-6, dtype=L.SPECFOLD_BF16)
        for _ in range(3):
            L.specfold_gate(sh, H, fs, 0.02, ratio, rec, stream)
        t0, t1 = ev.create(2)
        torch.cuda.synchronize()
        ev.record(t0, stream)
        for _ in range(reps):
            L.specfold_gate(sh, H, fs, 0.02, ratio, rec, stream)
        ev.record(t1, stream)
        torch.cuda.synchronize()
        us = ev.ms(t0, t1) / reps * 1e3
        ev.destroy([t0, t1])
        alg = S * d * 2 + S * 5
        issued = 2 * S * d * 2 - B * d * 2 + S * 5
        rows.append(dict(nodes=n, slots=S, hidden_bytes=S * d * 2, us=us,
                         GBps=alg / (us * 1e-6) / 1e9, hbm_frac=alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         issued_GBps=issued / (us * 1e-6) / 1e9))
        log(f"[bench] gate sweep {S * d * 2 / 1e6:.0f} MB: {us:.1f} us, "
            f"{rows[-1]['GBps']:.0f} GB/s ({rows[-1]['hbm_frac'] * 100:.0f}% of HBM peak), "
            f"{rows[-1]['issued_GBps']:.0f} GB/s of child+parent reads")
        del H, fs, ratio, rec
        torch.cuda.empty_cache()
    return rows


def budget_sweep(w1, ev, stream, steps, warmup):
    """Per-verify-layer time against the draft budget (the pages' Fig. 3 plots the
    per-verify latency rising with it): the 7B-shaped layer with 1 + {3, 7, 15, 31, 63}
    branches of one 3-ary level-order tree, dense (tau < 0, every branch recomputed) and
    folded at the configuration's tau.  Weights and prefix are those of the 1 + 15 layer
    (the same seed draws the same values); only the graph and the hidden states change."""
    import torch
    from branch_folding_amd.runner import DeviceLayer
    from synth import BUDGETS, budget_config, make_workload
    rows = []
    for n in BUDGETS:
        cfg = budget_config(n)
        wn = make_workload(cfg, layers=1, weights=False)
        dl = rotating(DeviceLayer(cfg, w1.weights[0], w1.cache, wn.H, wn.fold_src))
        for tau in (-1.0, cfg.tau):
            dl.forward(tau, stream=stream)
            torch.cuda.synchronize()
            K = dl.fold_state()["K"]
            ms, _ = time_layer(dl, tau, steps, warmup, ev, stream)
            rows.append(dict(branches=n, slots=cfg.slots, tau=tau, K=K,
                             recompute_fraction=K / cfg.slots, us=ms * 1e3,
                             branch_tokens_per_s=cfg.slots / (ms * 1e-3)))
            log(f"[bench] budget 1+{n - 1} tau={tau}: K={K} of {cfg.slots} "
                f"{ms * 1e3:.1f} us ({cfg.slots / (ms * 1e-3) / 1e6:.2f} M branch-tok/s)")
        del dl
        torch.cuda.empty_cache()
    return rows


def device_layers(cfg):
    """Per-layer weights and prefix caches of `cfg` drawn on the device (seeded torch
    generator, same distributions as the host generator: linear weights N(0, 0.02^2),
    RMSNorm gains 1, prefix K/V N(0, (0.02 sqrt(d))^2), rounded to bf16).  Drawing 13 GB
    of 28-layer weights on the host would take minutes; the timing does not depend on
    which seeded values the weights hold."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    d, f, dh = cfg.hidden, cfg.ffn, cfg.head_dim
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def lin(o, i):
        return (torch.randn(o, i, device="cuda", generator=g) * cfg.weight_std).to(dt)

    for _ in range(cfg.layers):
        w = {"rms1": torch.ones(d, device="cuda", dtype=dt), "w_qkv": lin(cfg.qkv_dim, d),
             "w_o": lin(d, cfg.n_q * dh), "rms2": torch.ones(d, device="cuda", dtype=dt),
             "w_gate_up": lin(2 * f, d), "w_down": lin(d, f)}
        cache = (torch.randn(cfg.prefix + 64, 2, cfg.n_kv, dh, device="cuda", generator=g)
                 * (0.02 * math.sqrt(d))).to(dt)
        yield w, cache


def stack_bench(ev, stream, steps, warmup):
    """End-to-end time of one verify step through the 28-layer 7B-shaped stack (1+31
    branches, prefix 4096): every layer gates, packs and runs on the previous layer's
    output inside one specfold_stack_forward call.  Hidden states and draft graph come
    from the host generator; weights and prefix caches are drawn on the device."""
    import torch
    from branch_folding_amd.runner import DeviceStack
    from synth import CONFIGS, make_workload
    cfg = CONFIGS[3]
    t = time.time()
    base = make_workload(cfg, layers=1, weights=False)
    ds = DeviceStack(cfg, device_layers(cfg), base.H, base.fold_src)
    torch.cuda.synchronize()
    log(f"[bench] stack {cfg.name}: {ds.num_layers} layers drawn on the device in "
        f"{time.time() - t:.1f}s")
    ds.forward(cfg.tau, stream=stream)
    torch.cuda.synchronize()
    Ks = [s["K"] for s in ds.fold_states()]
    for _ in range(warmup):
        ds.forward(cfg.tau, stream=stream, record_states=False)
    t0, t1 = ev.create(2)
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(steps):
        ds.forward(cfg.tau, stream=stream, record_states=False)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    log(f"[bench] stack: {ms * 1e3:.0f} us per verify step ({ms * 1e3 / ds.num_layers:.1f} "
        f"us per layer), K per layer {Ks}")
    # the same step captured as one HIP graph and replayed
    g = ds.capture(cfg.tau, record_states=False)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev.record(t0, stream)
    for _ in range(steps):
        g.replay()
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms_g = ev.ms(t0, t1) / steps
    ev.destroy([t0, t1])
    del g
    log(f"[bench] stack as one HIP graph: {ms_g * 1e3:.0f} us per verify step")
    res = dict(workload=cfg.name, layers=ds.num_layers, tau=cfg.tau, us_per_verify_step=ms * 1e3,
               us_per_layer=ms * 1e3 / ds.num_layers, packed_rows_per_layer=Ks,
               slots=cfg.slots, branch_tokens_per_s=cfg.slots / (ms * 1e-3),
               us_per_verify_step_graph=ms_g * 1e3,
               weights="drawn on the device: N(0, 0.02^2) linear weights, bf16")
    del ds
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
