"""Throughput of the MX MoE expert block on one MI355X, against the HBM / MFMA roofline.

One step = one mxmoe_forward call (route -> align -> MXFP8 quant -> gate_up + SwiGLU + requant ->
down + weighted combine -> bf16) over one batch of seeded synthetic input already resident in HBM.
Weights rotate through several device copies (together more than twice the 256 MB last-level
cache), so every step streams its expert weights from HBM as a serving loop does between calls of
the same layer; the cold-weight effect is the microbenchmark pitfall of "Ling-3.0-flash: Tối ưu hóa
độ trễ giải mã lên 54% trên 4 GPU Blackwell" ("Sửa thước đo trước khi sửa máy").

Prints one JSON line. `value` is the headline workload's algorithmic HBM throughput (GB/s) at
decode M; per-workload TFLOP/s, GB/s and roofline fractions (decode and prefill M) are in
`workloads`. `roofline` is for the dominant kernel (gate_up), timed with HIP events that the
library records on its own stream at stage boundaries. `cpu_baseline` is the fp64 CPU oracle on a
bounded sample of the headline workload (host cores of the same machine). `gate` times the router
gate in front of the block (mxmoe_gate, x . W_g^T to fp32 logits) on each workload's shapes, warm
(back-to-back calls) and cold (caches flushed before each call)."""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
# Dense MFMA peaks by the operand pair the block issues: bf16 2.5 PFLOP/s; 5.0 when either operand
# is E4M3 (MXFP8, and MXFP4 weights with MXFP8 activations run at the fp8 rate); 10.1 when both
# operands are E2M1 (MXFP4 weights with MXFP4 activations).
PEAK_MFMA_TFLOPS = {("bf16", "bf16"): 2500.0, ("mxfp8", "mxfp8"): 5000.0,
                    ("mxfp4", "mxfp8"): 5000.0, ("mxfp4", "mxfp4"): 10100.0}
LLC_BYTES = 256 << 20              # MALL (infinity cache)
METRIC = "MoE-block TFLOP/s and HBM GB/s (% of MI355X roofline) at decode/prefill M"
ELEM_BYTES = {"mxfp8": 1.0, "mxfp4": 0.5, "bf16": 2.0}


def mfma_peak(w):
    return PEAK_MFMA_TFLOPS[(w.w_fmt, w.act_fmt)]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- work figures
def expert_bytes(w, part="all"):
    """Algorithmic bytes of one expert's weights (codes + E8M0 scales)."""
    eb = ELEM_BYTES[w.w_fmt] + (0.0 if w.w_fmt == "bf16" else 1.0 / 32)
    per = {"w13": 2 * w.I * w.H * eb, "w2": w.H * w.I * eb}
    return per["w13"] + per["w2"] if part == "all" else per[part]


def block_bytes(w, touched):
    """Weights of the touched experts + x, logits and y (the block's own algorithmic traffic)."""
    return touched * expert_bytes(w) + w.T * w.H * 2 + w.T * w.E * 2 + w.T * w.H * 2


def gate_up_bytes(w, touched):
    act = ELEM_BYTES[w.act_fmt] + (0.0 if w.act_fmt == "bf16" else 1.0 / 32)   # codes + scales
    a_in = w.T * w.H * act
    h_out = w.slots * w.I * act
    return touched * expert_bytes(w, "w13") + a_in + h_out


def block_flops(w):
    return 6.0 * w.H * w.I * w.slots


def gate_up_flops(w):
    return 4.0 * w.H * w.I * w.slots


# ----------------------------------------------------------------------------- GPU leg
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)
STAGE_TIMING = ("mean over the stage-timing pass of a fence-free HIP event pair that the library "
                "records on its stream around the kernel")


class FenceFreeEvents:
    """n timing events of the HIP runtime already loaded in the process (torch's), created with
    hipEventDisableSystemFence: recording one skips the system-scope release, which is only
    needed when the host inspects the memory an event guards, so the interval between two of them
    is closer to the kernels' own time."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.handles[i] = h.value

    def elapsed_ms(self, i, j):
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), self.handles[i], self.handles[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy(self):
        for h in self.handles:
            self.hip.hipEventDestroy(h)


class GpuWorkload:
    def __init__(self, name, copies=None, threads=16):
        import torch
        import workloads
        from mx_quantized_grouped_amd import binding as B
        from mx_quantized_grouped_amd.weights import ExpertLoader
        self.torch, self.B = torch, B
        self.w = w = workloads.get(name)
        self.shape = B.Shape.of(w.T, w.H, w.E, w.top_k, w.I, w.w_fmt, act_fmt=w.act_fmt)
        t0 = time.time()
        loader = ExpertLoader(self.shape, "cuda")
        workloads.draw_all_experts(w, threads=threads, callback=loader.add_expert)
        packed = loader.finish()
        torch.cuda.synchronize()
        wbytes = sum(p.numel() for p in packed)
        n = copies or max(2, math.ceil(2 * LLC_BYTES / wbytes) + 1)
        self.packed = [packed] + [tuple(p.clone() for p in packed) for _ in range(n - 1)]
        torch.cuda.synchronize()
        log(f"{name}: weights {wbytes / 1e6:.1f} MB x {n} copies prepared in {time.time() - t0:.1f}s")
        to_dev = lambda b: torch.from_numpy(b.view(np.int16)).to("cuda").view(torch.bfloat16)
        self.xb, self.lb = workloads.draw_x(w), workloads.draw_logits(w)
        self.x, self.logits = to_dev(self.xb), to_dev(self.lb)
        self.y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
        self.ws = B.new_workspace(B.mxmoe_workspace_bytes(self.shape), "cuda")

    def step(self, i, options=None):
        self.B.mxmoe_forward(self.shape, self.x, self.logits, self.packed[i % len(self.packed)],
                             y=self.y, workspace=self.ws, options=options)

    def touched_experts(self):
        B = self.B
        off, nb, _ = B.mxmoe_workspace_view(self.shape, None, B.VIEW_TOPK_IDS)
        ids = self.ws[off:off + nb].view(self.torch.int32)
        return int(self.torch.unique(ids).numel())

    def time_steps(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            self.step(i)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps

    def time_graph(self, steps, warmup):
        """Average time of one forward per HIP graph replay: one graph per weight copy
        (captured once, replayed in the same rotation as the eager steps), so the launch overhead
        of the library's kernels is paid at capture, as a serving loop under graph execution
        would."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(self.packed)):
                self.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for i in range(len(self.packed)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record()
        torch.cuda.synchronize()
        del graphs
        return e0.elapsed_time(e1) / steps

    def time_each(self, steps):
        """Per-step durations from one event pair around each call (the pair's own cost included):
        the spread of the step time."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            a.record()
            self.step(i)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    def time_warm(self, steps):
        """Every call on the same weight copy (for context: whatever of it the caches keep)."""
        torch = self.torch
        for _ in range(3):
            self.step(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            self.step(0)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_stages(self, steps, fence_free=False):
        """Average duration of each stage, from events the library records on its stream.
        fence_free: events created with hipEventDisableSystemFence, whose record skips the
        system-scope release (an L2 write-back and invalidation); a default event pair around a
        short stage adds ~4 us of that to it."""
        torch, B = self.torch, self.B
        import ctypes
        n = B.MXMOE_STAGE_EVENTS
        if fence_free:
            evs = [FenceFreeEvents(n) for _ in range(steps)]
            arrs = [row.handles for row in evs]
        else:
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
            for row in evs:              # materialise the underlying hipEvent_t handles
                for e in row:
                    e.record()
            torch.cuda.synchronize()
            arrs = [(ctypes.c_void_p * n)(*[e.cuda_event for e in row]) for row in evs]
        for i in range(steps):
            opt = B.Options(0, 0, 0, 0, ctypes.cast(arrs[i], ctypes.POINTER(ctypes.c_void_p)))
            self.step(i, opt)
        torch.cuda.synchronize()
        out = {}
        for s, name in enumerate(B.STAGES):
            if fence_free:
                out[name] = float(np.mean([row.elapsed_ms(s, s + 1) for row in evs]))
            else:
                out[name] = float(np.mean([row[s].elapsed_time(row[s + 1]) for row in evs]))
        if fence_free:
            for row in evs:
                row.destroy()
        return out


def measure(name, steps, warmup):
    g = GpuWorkload(name)
    ms, wall_ms = g.time_steps(steps, warmup)
    each = g.time_each(max(10, min(steps, 50)))
    warm_ms = g.time_warm(max(10, min(steps, 50)))
    stages = g.time_stages(max(10, min(steps, 50)), fence_free=True)
    touched = g.touched_experts()
    w = g.w
    by = block_bytes(w, touched)
    fl = block_flops(w)
    res = {
        "T": w.T, "H": w.H, "E": w.E, "top_k": w.top_k, "shared_experts": 1, "I": w.I,
        "w_fmt": w.w_fmt, "act_fmt": w.act_fmt, "zipf": w.zipf, "touched_experts": touched,
        "ms_per_step": ms, "wall_ms_per_step": wall_ms,
        "step_ms_p10_p50_p90": [float(np.percentile(each, q)) for q in (10, 50, 90)],
        "warm_ms_per_step": warm_ms,
        "algorithmic_MB": by / 1e6, "GFLOP": fl / 1e9,
        "GBps": by / (ms * 1e-3) / 1e9, "TFLOPs": fl / (ms * 1e-3) / 1e12,
        "stage_ms": stages,
    }
    res["hbm_frac"] = res["GBps"] / PEAK_HBM_GBS
    res["mfma_frac"] = res["TFLOPs"] / mfma_peak(w)
    gu_ms = stages["gate_up"]
    decode = w.slots < 16 * (w.E + 1)
    if decode:   # decode sizes: the same steps replayed from HIP graphs
        gms = g.time_graph(steps, warmup)
        res["graph"] = {"ms_per_step": gms, "GBps": by / (gms * 1e-3) / 1e9,
                        "hbm_frac": by / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if decode:
        ach = gate_up_bytes(w, touched) / (gu_ms * 1e-3) / 1e9
        res["roofline"] = {"kernel": "gate_up", "bound": "hbm", "achieved": ach,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                           "bytes_per_launch": gate_up_bytes(w, touched),
                           "launch_us": gu_ms * 1e3, "timing": STAGE_TIMING}
    else:
        ach = gate_up_flops(w) / (gu_ms * 1e-3) / 1e12
        pk = mfma_peak(w)
        res["roofline"] = {"kernel": "gate_up", "bound": "mfma", "achieved": ach, "peak": pk,
                           "unit": "TFLOP/s", "frac": ach / pk, "flops_per_launch": gate_up_flops(w),
                           "launch_us": gu_ms * 1e3, "timing": STAGE_TIMING}
    log(f"{name}: {ms * 1e3:.1f} us/step, {res['GBps']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM), "
        f"{res['TFLOPs']:.1f} TFLOP/s ({100 * res['mfma_frac']:.1f}% MFMA), stages(us) "
        + ", ".join(f"{k}={v * 1e3:.1f}" for k, v in stages.items())
        + (f"; graph replay {res['graph']['ms_per_step'] * 1e3:.1f} us/step" if "graph" in res else "")
        + "; per-step p10/p50/p90 " + "/".join(f"{v * 1e3:.1f}" for v in res["step_ms_p10_p50_p90"])
        + f" us; warm {warm_ms * 1e3:.1f} us")
    return g, res


# ----------------------------------------------------------------------------- CPU baseline
def measure_gate(name, steps=100, cold_reps=30):
    """Router gate (mxmoe_gate, fp32 logits) on the workload's x [T, H] and a seeded bf16 gate
    [E, H]. Warm: launched back to back, its weights and activations staying in cache between
    calls. Cold: before each call a 512 MiB buffer is written (more than the 256 MB memory-side
    cache plus the eight 4 MB L2s), so x and the gate weights come from HBM, as between two layers
    of a serving step ("Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell",
    "Sửa thước đo trước khi sửa máy": 7 us hot against 11 us cold there); one event pair around
    each call, reported as the median, with the median of an empty pair for the events' own cost."""
    import torch
    import workloads
    from mx_quantized_grouped_amd import binding as B
    w = workloads.get(name)
    x = torch.from_numpy(workloads.draw_x(w).view(np.int16)).to("cuda").view(torch.bfloat16)
    gw = torch.from_numpy(workloads.draw_gate(w).view(np.int16)).to("cuda").view(torch.bfloat16)
    out = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    for _ in range(5):
        B.mxmoe_gate(x, gw, logits=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        B.mxmoe_gate(x, gw, logits=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold, empty = [], []
    for i in range(cold_reps):
        for timed in (True, False):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if timed:
                B.mxmoe_gate(x, gw, logits=out)
            b.record()
            torch.cuda.synchronize()
            (cold if timed else empty).append(a.elapsed_time(b) * 1e3)
    del flush
    nbytes = 2 * w.T * w.H + 2 * w.E * w.H + 4 * w.T * w.E
    cold_us = float(np.median(cold))
    return {"us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "TFLOPs": 2.0 * w.T * w.H * w.E / (us * 1e-6) / 1e12, "weights": "in cache",
            "cold_us": cold_us, "cold_GBps": nbytes / (cold_us * 1e-6) / 1e9,
            "cold_event_pair_us": float(np.median(empty)), "bytes": nbytes}


def cpu_baseline(g, n_tokens, min_seconds=10.0):
    """The fp64 oracle on a bounded sample: n_tokens tokens of the same workload. Weight codes are
    produced before the timed region (load-time work); the timed region is the block itself:
    routing, sort, Q1, explicit per-expert MX dequantisation, fp64 GEMMs, SwiGLU, Q2, combine."""
    import workloads
    from oracle import moe, mx
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = g.w
    toks = np.arange(min(n_tokens, w.T))
    x = workloads.f32_from_bf16_bits(g.xb).astype(np.float64)
    lg = workloads.f32_from_bf16_bits(g.lb).astype(np.float64)
    ids, _ = moe.route(lg[toks], w.top_k)
    need = sorted(set(ids.reshape(-1).tolist()))
    el = {"mxfp8": "e4m3", "mxfp4": "e2m1"}.get(w.w_fmt)
    def prep(e):                                      # untimed: load-time quantisation
        a, b = workloads.draw_expert(w, e)
        return e, ((mx.quantize(a, el), mx.quantize(b, el)) if el else (a, b))
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        coded = dict(ex.map(prep, need))

    def get(e):
        if not el:
            return np.asarray(coded[e][0], np.float64), np.asarray(coded[e][1], np.float64)
        (c13, s13), (c2, s2) = coded[e]
        return mx.dequantize(c13, s13, el), mx.dequantize(c2, s2, el)
    W = moe.ExpertWeights(w.E, w.H, w.I, w.w_fmt, get, cache=0)
    # the sample is repeated until about min_seconds of CPU work have been timed
    reps, total = 0, 0.0
    while reps < 1 or (total < min_seconds and reps < 200):
        t0 = time.perf_counter()
        r = moe.moe_block(x[toks], lg[toks], W, w.top_k, w.act_fmt)
        moe.align(r.ids, w.E, 16)
        total += time.perf_counter() - t0
        reps += 1
    sec = total / reps
    by = len(need) * expert_bytes(w) + len(toks) * (4 * w.H + 2 * w.E)
    y = g.y.float().cpu().numpy().astype(np.float64)[toks]
    par = moe.parity_stats(y, r.y)
    return {"value": by / sec / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": sec, "gflops": 6.0 * w.H * w.I * (w.top_k + 1) * len(toks) / sec / 1e9,
            "sample": f"{len(toks)} of {w.T} tokens of {w.name} ({len(need)} experts touched), "
                      f"timed {reps} times ({total:.1f} s of CPU work); fp64 numpy, same process "
                      f"and host",
            "parity_vs_gpu_on_sample": par}


GEMM_SOURCES = ("gemm.hip", "gemm_dev.h", "device.h")   # the sources the GEMM kernels compile from


def gemm_source_hash():
    """sha256 (16 hex digits) over the GEMM kernels' sources, in a fixed order."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "mx_quantized_grouped_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record(name):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else null)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(name)
    if not rec:
        return None
    return rec.get("bytes_per_launch") if rec.get("gemm_src_sha") == gemm_source_hash() else None


def sweep_launchers(specs, tokens, steps=10, warmup=3):
    """Forward time of the small-M and the large-M launcher (and the automatic plan) over batch
    sizes, with cold weights as in `measure`. specs: workload names, each optionally suffixed
    ':uniform' or ':zipf' to set the routing; the workload's other sizes are kept and T varies.
    Prints one line per (spec, T) to stderr and returns the rows."""
    import dataclasses
    import torch
    import workloads
    from mx_quantized_grouped_amd import binding as B
    rows = []
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).to("cuda").view(torch.bfloat16)
    for spec in specs:
        base, _, routing = spec.partition(":")
        g = GpuWorkload(base)
        w0 = g.w if not routing else dataclasses.replace(g.w, zipf=routing == "zipf")
        for T in tokens:
            w = dataclasses.replace(w0, T=T)
            shape = B.Shape.of(T, w.H, w.E, w.top_k, w.I, w.w_fmt, act_fmt=w.act_fmt)
            x, lg = to_dev(workloads.draw_x(w)), to_dev(workloads.draw_logits(w))
            y = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
            res = {}
            for tag, opt in [("small", B.Options(1, 0, 0, 0)), ("large", B.Options(2, 0, 0, 0)),
                             ("auto", None)]:
                ws = B.new_workspace(B.mxmoe_workspace_bytes(shape, opt), "cuda")
                for i in range(warmup):
                    B.mxmoe_forward(shape, x, lg, g.packed[i % len(g.packed)], y=y, workspace=ws,
                                    options=opt)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(steps):
                    B.mxmoe_forward(shape, x, lg, g.packed[i % len(g.packed)], y=y, workspace=ws,
                                    options=opt)
                e1.record()
                torch.cuda.synchronize()
                res[tag] = e0.elapsed_time(e1) / steps * 1e3
                del ws
            r = {"spec": spec, "T": T, "slots_per_expert": T * (w.top_k + 1) / (w.E + 1),
                 "small_us": res["small"], "large_us": res["large"], "auto_us": res["auto"]}
            rows.append(r)
            log(f"sweep {spec} T={T} S/(E+1)={r['slots_per_expert']:.1f}: small {res['small']:.1f}, "
                f"large {res['large']:.1f}, auto {res['auto']:.1f} us")
        del g
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_mxfp8")
    ap.add_argument("--extra", default="prefill_mxfp8,decode_mxfp4,wide512_mxfp4_T1,"
                                       "wide512_mxfp4_T6,wide512_mxfp4_T4096,decode_w4a4,"
                                       "wide512_w4a4_T4096",
                    help="comma-separated extra workloads, 'all', or 'none'")
    ap.add_argument("--cpu-tokens", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run three device-to-device copies of this many MiB (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    ap.add_argument("--sweep-launchers", default="",
                    help="instead of the bench line: comma-separated workloads (optionally "
                         "':uniform' / ':zipf') to time with both launchers over --sweep-tokens")
    ap.add_argument("--sweep-tokens", default="32,64,128,192,224,256,288,320,352,384,512,768,1024,"
                                              "1536,2048,4096")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block runs on one GPU's share of the tensor-parallel "
              "shapes and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from mx_quantized_grouped_amd import binding as B
    B.lib()
    if args.sweep_launchers:
        rows = sweep_launchers(args.sweep_launchers.split(","),
                               [int(v) for v in args.sweep_tokens.split(",")])
        print(json.dumps({"launcher_sweep": rows}), flush=True)
        return
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.calibrate_copy_mb} MiB device-to-device")
        del src, dst
        torch.cuda.empty_cache()
    g, head = measure(args.workload, args.steps, args.warmup)
    others = {}
    extra = [] if args.extra == "none" else (
        [n for n in workloads.WORKLOADS if n != args.workload] if args.extra == "all"
        else [n for n in args.extra.split(",") if n and n != args.workload])
    base = None if args.no_cpu_baseline else cpu_baseline(g, args.cpu_tokens)
    del g
    torch.cuda.empty_cache()
    for n in extra:
        gx, r = measure(n, max(10, args.steps // 2), max(3, args.warmup // 2))
        others[n] = r
        del gx
        torch.cuda.empty_cache()
    gate_shapes = {}
    for n in [args.workload] + extra:   # one gate measurement per (T, H, E)
        wn = workloads.get(n)
        gate_shapes.setdefault((wn.T, wn.H, wn.E), n)
    gate = {n: measure_gate(n) for n in gate_shapes.values()}
    rl = dict(head["roofline"])
    rl["traffic"] = traffic_record(args.workload)
    w = workloads.get(args.workload)
    out = {
        "metric": METRIC, "value": head["GBps"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->f32" if w.w_fmt == "bf16" else f"{w.w_fmt}x{w.act_fmt}->f32",
        "data": "synthetic (seeded draws; weights N(0,0.02) quantised on the GPU)",
        "config": {"workload": args.workload, **{k: head[k] for k in
                   ("T", "H", "E", "top_k", "shared_experts", "I", "w_fmt", "act_fmt", "zipf")},
                   "parallelism": "single GPU (one TP share, all experts resident)"},
        "tflops": head["TFLOPs"], "hbm_frac": head["hbm_frac"], "mfma_frac": head["mfma_frac"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"], "warm_ms_per_step": head["warm_ms_per_step"],
        "touched_experts": head["touched_experts"], "stage_ms": head["stage_ms"],
        "roofline": rl, "cpu_baseline": base, "graph": head.get("graph"), "gate": gate,
        "workloads": {n: {k: v for k, v in r.items() if k not in ("T", "H", "E", "top_k",
                                                                  "shared_experts")}
                      for n, r in others.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
