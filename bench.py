"""Throughput of the MoE layout -> dispatch -> combine path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is the whole path over one batch of the 8K-token workload
(T=8192 tokens, hidden 7168, 256 experts in 8 ranks, top-8 group-limited
routing): ep_layout, FP8 E4M3 1x128 ep_dispatch and BF16 ep_combine, all on
one HIP stream with every input already resident in HBM.  The headline value
is algorithmic bytes per step (layout + dispatch + combine, counted as the
method must move them) times K over the wall time of K steps.

Also reported: per-stage kernel times from HIP events recorded around each
call in a second timed loop (mean, median, p10, p90), the roofline of the
dominant kernel (combine, HBM-bound), the same step "cold" (each step after
reading a 1 GiB buffer, so no cache holds its data), the decode-shaped
workload's microseconds per call, the same step with layout and dispatch as
one ep_layout_dispatch call, the backward pair's kernel times on the
same handle, dispatch in every receive format (BF16, FP8, MXFP8, MXFP4,
pre-quantised FP8), warm and cold step times of the tiny, mid
and 16K-token skewed workloads, a plain 1 GiB copy and a streaming probe
at each stage's own read:write mix as practical bandwidth ceilings, and the
CPU oracle timed on this host (one thread, and all usable cores, with the
CPU model) on the same workload.

Prints exactly one JSON line on stdout; progress goes to stderr.

Measured HBM traffic of the combine kernel comes from two rocprofv3 counter
runs of this script (FETCH_SIZE, then WRITE_SIZE) with --calibration-copy,
which adds a plain 1 GiB device copy whose true byte counts scale the
counters:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d F -- python3 bench.py --steps 3 --warmup 1 --no-decode --no-configs --no-extras --no-cpu-baseline --calibration-copy
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d W -- python3 bench.py --steps 3 --warmup 1 --no-decode --no-configs --no-extras --no-cpu-baseline --calibration-copy
    python3 bench.py --traffic-from F W

The last command writes profiles/combine_v3_traffic.json, stamped with a hash
of the combine kernel's source; the traffic figure is reported only while
that source is unchanged.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import combine_ep_layout_02_amd as ep  # noqa: E402
from combine_ep_layout_02_amd import ep as epmod  # noqa: E402
from combine_ep_layout_02_amd import workloads as wl  # noqa: E402

METRIC = "dispatch+combine HBM GB/s & % peak at 8K tok,h7168,top-8; decode µs/call"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_v3_traffic.json")
KERNEL_SOURCES = ["combine_ep_layout_02_amd/csrc/ep_combine.hip", "combine_ep_layout_02_amd/csrc/ep_device.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# algorithmic bytes (what the method must move)
# --------------------------------------------------------------------------

def bytes_layout(w):
    return 8 * w.num_tokens * w.num_topk + 4 * w.recv_rows


def bytes_dispatch(w, fp8):
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    if fp8:
        return 2 * T * H + 4 * T * k + T * k * H + 4 * T * k * (H // 128)
    return 2 * T * H + 4 * T * k + 2 * T * k * H


def bytes_dispatch_format(w, fmt):
    """Algorithmic bytes of one dispatch call in each receive format."""
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    base = 2 * T * H + 4 * T * k                       # read x and the slots
    return base + {"bf16": 2 * T * k * H,
                   "fp8": T * k * H + 4 * T * k * (H // 128),
                   "mxfp8": T * k * H + T * k * (H // 32),
                   "mxfp4": T * k * H // 2 + T * k * (H // 32),
                   "fp8_prequantized": T * k * H + 4 * T * k * (H // 128) - T * H + 4 * T * (H // 128)}[fmt]


def bytes_combine(w):
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    return 2 * T * k * H + 8 * T * k + 2 * T * H


def bytes_dispatch_backward(w):
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    return 2 * T * k * H + 4 * T * k + 2 * T * H


def bytes_combine_backward(w):
    T, H, k = w.num_tokens, w.hidden, w.num_topk
    return 2 * T * H + 4 * T * k * H + 12 * T * k


# --------------------------------------------------------------------------
# device setup
# --------------------------------------------------------------------------

class Step:
    """Device buffers of one workload and the three calls of one step."""

    def __init__(self, w, dev, fp8=True):
        self.w, self.fp8 = w, fp8
        self.shape = ep.EpShape(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                                w.expert_alignment, w.capacity)
        inp = wl.make_inputs(w)
        self.inp = inp
        self.idx = torch.from_numpy(inp.topk_idx).to(dev)
        self.wts = torch.from_numpy(inp.topk_weights).to(dev)
        self.x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.y = torch.from_numpy(inp.y.view(np.int16)).to(dev).view(torch.bfloat16)
        self.lay = ep.LayoutBuffers.allocate(self.shape, dev)
        self.dtype = ep.EP_FP8_E4M3 if fp8 else ep.EP_BF16
        self.recv_x, self.recv_scale = ep.alloc_recv(self.shape, self.dtype, dev)
        self.out = torch.empty_like(self.x)
        # argument checks and the stream lookup once; the timed loop only launches
        stream = torch.cuda.current_stream(dev)
        self.layout = self.lay.prepare(self.idx, stream)
        self.dispatch = ep.prepare_dispatch(self.shape, self.x, self.lay.slot, self.dtype, self.recv_x,
                                            self.recv_scale, stream)
        self.combine = ep.prepare_combine(self.shape, self.y, self.lay.slot, self.wts, self.out, stream)
        # layout and dispatch as one call (one launch for batches of at most 1024 pairs)
        self.layout_dispatch = self.lay.prepare_dispatch(self.idx, self.x, self.dtype, self.recv_x, self.recv_scale,
                                                         stream)

    def run(self):
        self.layout()
        self.dispatch()
        self.combine()

    def run_fused(self):
        self.layout_dispatch()
        self.combine()

    @property
    def bytes(self):
        return bytes_layout(self.w) + bytes_dispatch(self.w, self.fp8) + bytes_combine(self.w)


def time_steps(step, steps, warmup, fused=False):
    """Warm up, then time `steps` back-to-back steps between two HIP events on
    the launch stream (torch's current stream, which the binding launches on)."""
    run = step.run_fused if fused else step.run
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        run()
    end.record()
    step.submit_s = time.perf_counter() - t0   # host time to enqueue the steps
    torch.cuda.synchronize()
    return start.elapsed_time(end), time.perf_counter() - t0


def time_stages(step, steps, flush=None):
    """Per-stage kernel time: HIP events around each call, on the launch stream.
    With `flush`, it runs before each step, outside the events."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        if flush is not None:
            flush()
        e[0].record()
        step.layout()
        e[1].record()
        step.dispatch()
        e[2].record()
        step.combine()
        e[3].record()
    torch.cuda.synchronize()
    return np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])  # ms


class ReadFlush:
    """Reads a 1 GiB buffer (an fp32 sum into one value): afterwards the
    256 MB Infinity Cache and the L2s hold clean lines of that buffer, none
    of the step's data, and there is no dirty data whose write-back the next
    step would pay for (as there would be after writing the buffer).  The
    sum is taken in the buffer's own dtype: asking for another one would
    first write a converted copy."""

    def __init__(self, dev):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        self.sink.copy_(self.buf.sum())


def time_cold(step, reps, flush):
    """Whole-step time after a cache flush: two events around each step."""
    ms = []
    torch.cuda.synchronize()
    for _ in range(reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step.run()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return np.array(ms)


def time_backward(step, reps):
    """The backward pair on the step's handle: dispatch backward of a gradient
    shaped like the received rows, combine backward of an output gradient
    (with the gate-weight gradient).  Events around each call."""
    w, dev = step.w, step.x.device
    stream = torch.cuda.current_stream(dev)
    grad_recv = step.y                       # any BF16 [rows, H] buffer serves as the gradient
    grad_x = torch.empty_like(step.x)
    grad_out = step.x                        # and any BF16 [T, H] one as the output gradient
    grad_y = torch.empty_like(step.y)
    grad_w = torch.empty_like(step.wts)
    dbw = ep.prepare_dispatch_backward(step.shape, grad_recv, step.lay.slot, grad_x, stream)
    cbw = ep.prepare_combine_backward(step.shape, grad_out, step.y, step.lay.slot, step.wts, grad_y, grad_w,
                                      stream)
    meds = []
    for fn in (dbw, cbw):   # each in a loop of its own: steady state of that kernel alone
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        meds.append(float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3)
    d_us, c_us = meds
    db, cb = bytes_dispatch_backward(w), bytes_combine_backward(w)
    return {"dispatch_backward": {"us": round(float(d_us), 2), "bytes": db, "GBps": round(db / d_us / 1e3, 1)},
            "combine_backward": {"us": round(float(c_us), 2), "bytes": cb, "GBps": round(cb / c_us / 1e3, 1)},
            "note": f"medians of {reps} back-to-back calls of each with events around each call, on the "
                    "step's routing handle; combine_backward includes the gate-weight gradient"}


def cu_sweep(dev, budgets, gemm_n=4096, reps=10):
    """Dispatch (FP8) and combine on the 8192-token workload under CU budgets
    (ep_shape_t.num_cus): alone, and beside a BF16 GEMM stream standing in for
    the expert computation the pages overlap communication with.  0 = the
    whole GPU."""
    w = wl.WORKLOADS["v3"]
    step = Step(w, dev, fp8=True)
    step.run()
    s_ep = torch.cuda.current_stream(dev)
    s_mm = torch.cuda.Stream(dev)        # default priority, like every stream here
    a = torch.randn((w.num_tokens, w.hidden), device=dev).to(torch.bfloat16)
    b = torch.randn((w.hidden, gemm_n), device=dev).to(torch.bfloat16)
    c = torch.empty((w.num_tokens, gemm_n), device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gemm_flop = 2.0 * w.num_tokens * w.hidden * gemm_n

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def gemms(n):
        for _ in range(n):
            torch.matmul(a, b, out=c)

    # GEMM alone: enough GEMMs to cover the EP work of one measurement
    with torch.cuda.stream(s_mm):
        gemms(3)
        e0, e1 = ev(), ev()
        e0.record()
        gemms(20)
        e1.record()
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1) / 20
    rows = []
    for n in budgets:
        shape = dataclasses.replace(step.shape, num_cus=n)
        disp = ep.prepare_dispatch(shape, step.x, step.lay.slot, step.dtype, step.recv_x, step.recv_scale, s_ep)
        comb = ep.prepare_combine(shape, step.y, step.lay.slot, step.wts, step.out, s_ep)
        disp()
        comb()
        torch.cuda.synchronize()
        # alone
        t = []
        for fn in (disp, comb):
            e = [(ev(), ev()) for _ in range(reps)]
            for x0, x1 in e:
                x0.record(s_ep)
                fn()
                x1.record(s_ep)
            torch.cuda.synchronize()
            t.append(float(np.median([x0.elapsed_time(x1) for x0, x1 in e])))
        alone_ms = t[0] + t[1]
        # beside the GEMM stream: EP pairs on s_ep while GEMMs run on s_mm
        n_gemm = max(2, int(round(reps * alone_ms / gemm_ms)))
        g0, g1, p0, p1 = ev(), ev(), ev(), ev()
        torch.cuda.synchronize()
        g0.record(s_mm)
        with torch.cuda.stream(s_mm):
            gemms(n_gemm)
        g1.record(s_mm)
        p0.record(s_ep)
        for _ in range(reps):
            disp()
            comb()
        p1.record(s_ep)
        torch.cuda.synchronize()
        ep_ms = p0.elapsed_time(p1) / reps
        mm_ms = g0.elapsed_time(g1)
        both_ms = max(g0.elapsed_time(g1), g0.elapsed_time(p1))
        serial_ms = n_gemm * gemm_ms + reps * alone_ms
        rows.append({
            "num_cus": n,
            "dispatch_us": round(t[0] * 1e3, 1), "combine_us": round(t[1] * 1e3, 1),
            "dispatch_GBps": round(bytes_dispatch(w, True) / t[0] / 1e6, 1),
            "combine_GBps": round(bytes_combine(w) / t[1] / 1e6, 1),
            "with_gemm": {"ep_pair_us": round(ep_ms * 1e3, 1),
                          "ep_GBps": round((bytes_dispatch(w, True) + bytes_combine(w)) / ep_ms / 1e6, 1),
                          "gemm_TFLOPs": round(n_gemm * gemm_flop / mm_ms / 1e9, 1),
                          "gemms": n_gemm, "overlap_speedup": round(serial_ms / both_ms, 3)},
        })
        log(f"[cu-sweep] {rows[-1]}")
    return {"workload": "v3 (8192 tokens, hidden 7168, top-8; FP8 dispatch, BF16 combine)",
            "gemm": f"torch.matmul bf16 [{w.num_tokens}, {w.hidden}] x [{w.hidden}, {gemm_n}] on a second stream",
            "gemm_alone_TFLOPs": round(gemm_flop / gemm_ms / 1e9, 1), "gemm_alone_us": round(gemm_ms * 1e3, 1),
            "rows": rows,
            "note": "num_cus = persistent workgroups of up to 1024 threads (0 = one wavefront per work item); "
                    "ep_pair_us is dispatch + combine per pair while the GEMM stream runs; overlap_speedup = "
                    "(GEMMs alone + pairs alone) / (both streams together)"}


def time_formats(step, reps):
    """Dispatch of the step's tokens in every receive format, on its handle."""
    w, dev = step.w, step.x.device
    stream = torch.cuda.current_stream(dev)
    shape = step.shape
    T, H = w.num_tokens, w.hidden
    calls = {}
    for fmt, dt in (("bf16", ep.EP_BF16), ("fp8", ep.EP_FP8_E4M3), ("mxfp8", ep.EP_MXFP8_E4M3),
                    ("mxfp4", ep.EP_MXFP4_E2M1)):
        rx, rs = ep.alloc_recv(shape, dt, dev)
        calls[fmt] = ep.prepare_dispatch(shape, step.x, step.lay.slot, dt, rx, rs, stream)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    ident = ep.EpShape(T, H, 1, w.num_experts, w.num_ranks)
    ep.ep_dispatch(ident, step.x, torch.arange(T, dtype=torch.int32, device=dev)[:, None], ep.EP_FP8_E4M3, xq, xs)
    rq, rs = ep.alloc_recv(shape, ep.EP_FP8_E4M3, dev)
    calls["fp8_prequantized"] = ep.prepare_dispatch_prequantized(shape, xq, xs, step.lay.slot, rq, rs, stream)
    out = {}
    for fmt, fn in calls.items():
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        nbytes = bytes_dispatch_format(w, fmt)
        out[fmt] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1)}
    del calls
    torch.cuda.empty_cache()
    out["note"] = (f"dispatch of the {w.num_tokens}-token batch on the step's handle, median of {reps} calls; "
                   "mxfp8/mxfp4 carry one E8M0 scale per 32 columns, fp8 one fp32 scale per 128; "
                   "fp8_prequantized scatters caller-quantised codes and scales")
    return out


def pct(a, q):
    return round(float(np.percentile(a, q)) * 1e3, 2)


def spread_us(a):
    """median, p10 and p90 of times in ms, as microseconds."""
    return {"median": pct(a, 50), "p10": pct(a, 10), "p90": pct(a, 90)}


def summarize_config(w, fp8, dev, steps, flush):
    """Warm (back-to-back) and cold (flushed) step time of one more workload."""
    step = Step(w, dev, fp8=fp8)
    total_ms, _ = time_steps(step, steps, 5)
    fused_ms, _ = time_steps(step, steps, 5, fused=True)
    cold = time_cold(step, 10, flush)
    nbytes = step.bytes
    warm_us = total_ms / steps * 1e3
    fused_us = fused_ms / steps * 1e3
    cold_us = float(np.median(cold)) * 1e3
    return {"dispatch": "fp8_e4m3" if fp8 else "bf16", "tokens": w.num_tokens, "hidden": w.hidden,
            "experts": w.num_experts, "topk": w.num_topk, "capacity": w.capacity, "bytes_per_step": nbytes,
            "warm_us": round(warm_us, 2), "warm_GBps": round(nbytes / warm_us / 1e3, 1),
            "warm_us_layout_dispatch_call": round(fused_us, 2),
            "cold_us": round(cold_us, 2), "cold_GBps": round(nbytes / cold_us / 1e3, 1)}


def source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per combine launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


# --------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------

def calibration_copy(dev, reps=3):
    """A plain streaming elementwise kernel of exactly 1 GiB read and 1 GiB written
    (bitwise NOT of 2^29 int16); returns its median GB/s (read + written bytes)."""
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.bitwise_not(a, out=b)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del a, b
    return 2 * (1 << 30) / (float(np.median(ms)) / 1e3) / 1e9


def mix_ceilings(step, reps=10):
    """The streaming probe (ep_probe_stream: contiguous 1 KiB chunks, no gathers)
    at each stage's own read:write byte mix, on the step's own buffers, under
    each of its four cache policies, in round-robin and in XCD-contiguous unit
    order; the best is the practical ceiling of a plain copy with that mix on
    this machine.  Overwrites the step's outputs; run after the timed legs."""
    res = {}
    policies = ("nt/nt", "default/default", "nt/sc1", "default/nt")
    policies = policies + tuple(p + " xcd" for p in policies)  # + 4: units in XCD-contiguous order
    # combine reads 8 bytes per byte written (y rows -> out); FP8 dispatch writes ~4 per byte read (x -> recv_x)
    for name, src, dst, r, wr in (("combine", step.y, step.out, 16, 2), ("dispatch", step.x, step.recv_x, 2, 8)):
        units = min(src.numel() * src.element_size() // (r * 1024), dst.numel() * dst.element_size() // (wr * 1024))
        nbytes = units * (r + wr) * 1024
        per = {}
        for pol, pname in enumerate(policies):
            ms = []
            for _ in range(reps + 2):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                ep.ep_probe_stream(src, dst, units, r, wr, pol)
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            per[pname] = round(nbytes / (float(np.median(ms[2:])) / 1e3) / 1e9, 1)
        best = max(per, key=per.get)
        res[name] = {"read_KiB_per_unit": r, "write_KiB_per_unit": wr, "units": units, "bytes": nbytes,
                     "GBps": per[best], "policy": best, "GBps_by_policy": per}
    return res


def host_cpu():
    """Model name and usable cores of the host that runs the CPU oracle."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "usable_cores": len(os.sched_getaffinity(0)), "logical_cpus": os.cpu_count()}


def traffic_from(fetch_dir, write_dir):
    """Combine-kernel HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    each scaled by what the same counter reads for the 1 GiB calibration copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        out = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = "combine" if "combine_kernel" in name else "copy" if "bitwise_not" in name else None
                if key:
                    out.setdefault(key, []).append(float(r["Counter_Value"]))
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    f_scale = gib_kib / float(np.median(fetch["copy"]))
    w_scale = gib_kib / float(np.median(write["copy"]))
    fb = float(np.median(fetch["combine"])) * f_scale * 1024
    wb = float(np.median(write["combine"])) * w_scale * 1024
    rec = {"kernel": "combine_kernel<8, nt loads, sc1 stores> on the 8192-token workload", "source_hash": source_hash(),
           "fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
           "algorithmic_bytes_per_launch": bytes_combine(wl.WORKLOADS["v3"]),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "raw_fetch_kib": float(np.median(fetch["combine"])), "raw_write_kib": float(np.median(write["combine"])),
           "copy_fetch_kib": float(np.median(fetch["copy"])), "copy_write_kib": float(np.median(write["copy"]))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(step):
    import oracle  # test infrastructure; only this leg of the benchmark uses it
    w, inp = step.w, step.inp
    times = []
    for _ in range(2):
        t0 = time.perf_counter()
        lay = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment, w.capacity)
        oracle.dispatch_fp8(inp.x, lay.slot, w.recv_rows)
        oracle.combine(inp.y, lay.slot, inp.topk_weights)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(step.bytes / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the full {w.name} step (layout + FP8 dispatch + combine of {w.num_tokens} tokens), "
                      f"median of 2 runs, {t:.2f} s each, single-threaded C on the host"}


def cpu_baseline_parallel(step, threads):
    """The same oracle functions on all the host's cores: the layout (a single
    sequential counting sort) on one thread, then dispatch and combine on
    contiguous token ranges, one per thread (ctypes releases the GIL)."""
    import oracle  # test infrastructure; only this leg of the benchmark uses it
    from concurrent.futures import ThreadPoolExecutor
    w, inp = step.w, step.inp
    T = w.num_tokens
    q = np.zeros((w.recv_rows, w.hidden), np.uint8)
    sc = np.zeros((w.recv_rows, w.hidden // 128), np.float32)
    out = np.zeros((T, w.hidden), np.uint16)
    bounds = [(T * i // threads, T * (i + 1) // threads) for i in range(threads)]
    times = []
    with ThreadPoolExecutor(threads) as pool:
        for _ in range(3):
            t0 = time.perf_counter()
            lay = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment, w.capacity)
            list(pool.map(lambda b: oracle.dispatch_fp8(inp.x[b[0]:b[1]], lay.slot[b[0]:b[1]], w.recv_rows, (q, sc)),
                          bounds))
            list(pool.map(lambda b: oracle.combine(inp.y, lay.slot[b[0]:b[1]], inp.topk_weights[b[0]:b[1]],
                                                   out[b[0]:b[1]]), bounds))
            times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(step.bytes / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full {w.name} step, layout on one thread, dispatch and combine split by tokens over "
                      f"{threads} threads, median of 3 runs, {t:.3f} s each"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3", choices=["v3", "skew"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the backward pair and the other dispatch formats")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, mid and 16K-token skewed workloads")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="counter runs: keep the 1 GiB calibration copy to 3 launches")
    ap.add_argument("--cu-sweep", nargs="*", type=int, metavar="N",
                    help="instead of the benchmark: dispatch and combine under CU budgets N (0 = whole GPU), "
                         "alone and beside a GEMM stream; prints one JSON line")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 counter runs into profiles/combine_v3_traffic.json and exit")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the path; it has no multi-GPU mode "
              "(the ranks are segments of one HBM buffer). Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(epmod.library_path()):
        from combine_ep_layout_02_amd.build import build_library
        build_library()
    dev = torch.device("cuda:0")
    if args.cu_sweep is not None:
        budgets = args.cu_sweep or [8, 16, 32, 48, 64, 96, 128, 192, 256, 0]
        print(json.dumps(cu_sweep(dev, budgets)), flush=True)
        return

    w = wl.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} inputs")
    step = Step(w, dev, fp8=True)
    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up")
    total_ms, wall = time_steps(step, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    value = step.bytes * args.steps / (total_ms / 1e3) / 1e9
    stage = time_stages(step, args.steps)
    lay_ms, disp_ms, comb_ms = stage.mean(axis=0)
    # the same step with layout and dispatch as one call (ep_layout_dispatch)
    fused_ms, _ = time_steps(step, args.steps, args.warmup, fused=True)
    fused_us = fused_ms / args.steps * 1e3
    log("[bench] cold steps (1 GiB read before each)")
    flush = ReadFlush(dev)
    cold_step = time_cold(step, 20, flush)
    cold_stage = time_stages(step, 20, flush)
    cold_us = float(np.median(cold_step)) * 1e3

    backward = formats = None
    if not args.no_extras:
        log("[bench] backward pair")
        backward = time_backward(step, 20)
        log("[bench] dispatch formats")
        formats = time_formats(step, 20)

    dec = None
    if not args.no_decode:
        log("[bench] decode workload")
        dstep = Step(wl.WORKLOADS["decode"], dev, fp8=True)
        n = 500
        d_total, _ = time_steps(dstep, n, 50, fused=True)
        d_submit = dstep.submit_s
        d_unfused, _ = time_steps(dstep, n, 50)
        d_stage = time_stages(dstep, 100)
        dec = {"us_per_call": round(d_total / n * 1e3, 2),
               "us_per_call_separate_layout": round(d_unfused / n * 1e3, 2),
               "host_enqueue_us_per_call": round(d_submit / n * 1e6, 2),
               "layout_us": round(float(np.median(d_stage[:, 0])) * 1e3, 2),
               "dispatch_us": round(float(np.median(d_stage[:, 1])) * 1e3, 2),
               "combine_us": round(float(np.median(d_stage[:, 2])) * 1e3, 2),
               "bytes": dstep.bytes,
               "note": "one call = layout + FP8 dispatch (ep_layout_dispatch: one launch for this 1024-pair batch) "
                       "+ combine of 128 tokens into the padded [256, 128, 7168] layout; mean over 500 back-to-back "
                       "calls (inputs stay in the 256 MB Infinity Cache); us_per_call_separate_layout runs "
                       "ep_layout and ep_dispatch as two launches; stage times are medians with events around "
                       "each kernel of the two-launch form"}
        del dstep

    configs = None
    if not args.no_configs:
        configs = {}
        others = [("tiny", False), ("tiny", True), ("mid", False),
                  ("skew" if w.name != "skew" else "v3", True)]
        for name, fp8 in others:
            log(f"[bench] {name} {'fp8' if fp8 else 'bf16'}")
            configs[f"{name}_{'fp8' if fp8 else 'bf16'}"] = summarize_config(wl.WORKLOADS[name], fp8, dev, 20, flush)
            torch.cuda.empty_cache()
    del flush

    log("[bench] mix ceilings")
    mix = mix_ceilings(step)
    copy_gbps = calibration_copy(dev, reps=3 if args.calibration_copy else 5)
    cb = cbp = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle")
        cb = cpu_baseline(step)
        cbp = cpu_baseline_parallel(step, max(1, min(16, len(os.sched_getaffinity(0)))))

    comb_bytes = bytes_combine(w)
    achieved = comb_bytes / (comb_ms / 1e3) / 1e9
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.num_tokens} tokens, hidden={w.hidden}, E={w.num_experts} "
                               f"experts in {w.num_ranks} virtual ranks, top-{w.num_topk} group-limited routing, "
                               f"FP8 E4M3 1x128-scaled dispatch, BF16 combine",
                   "tokens": w.num_tokens, "hidden": w.hidden, "experts": w.num_experts,
                   "ranks": w.num_ranks, "topk": w.num_topk, "dispatch": "fp8_e4m3", "combine": "bf16",
                   "bytes_per_step": step.bytes},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "stages_us": {"layout": round(float(lay_ms) * 1e3, 2), "dispatch": round(float(disp_ms) * 1e3, 2),
                      "combine": round(float(comb_ms) * 1e3, 2)},
        "stage_GBps": {"dispatch": round(bytes_dispatch(w, True) / (disp_ms / 1e3) / 1e9, 1),
                       "combine": round(achieved, 1)},
        "stages_spread_us": {n: spread_us(stage[:, i]) for i, n in enumerate(("layout", "dispatch", "combine"))},
        "layout_dispatch_call": {"step_us": round(fused_us, 2), "GBps": round(step.bytes / fused_us / 1e3, 1),
                                 "note": "the same step with ep_layout_dispatch for layout + dispatch, then "
                                         "ep_combine; at this size it enqueues the layout and dispatch launches"},
        "cold": {"step_us": spread_us(cold_step), "GBps": round(step.bytes / cold_us / 1e3, 1),
                 "pct_of_hbm_peak": round(100 * step.bytes / cold_us / 1e3 / HBM_PEAK_GBS, 2),
                 "stages_us": {n: spread_us(cold_stage[:, i])
                               for i, n in enumerate(("layout", "dispatch", "combine"))},
                 "note": "20 steps, each after reading a 1 GiB buffer, so that neither the Infinity Cache nor "
                         "the L2s hold any of the step's data"},
        "roofline": {"kernel": "combine", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": comb_bytes,
                     "mix_ceiling_GBps": mix["combine"]["GBps"],
                     "frac_of_mix_ceiling": round(achieved / mix["combine"]["GBps"], 4)},
        "mix_ceilings": dict(mix, note="ep_probe_stream at each stage's read:write mix (contiguous 1 KiB chunks, no "
                                       "gathers) on the step's buffers, best of four cache policies x two unit orders; *_frac = the "
                                       "stage's GB/s over it",
                             combine_frac=round(achieved / mix["combine"]["GBps"], 4),
                             dispatch_frac=round(bytes_dispatch(w, True) / (disp_ms / 1e3) / 1e9
                                                 / mix["dispatch"]["GBps"], 4)),
        "copy_ceiling": {"GBps": round(copy_gbps, 1), "kernel": "torch bitwise_not, 1 GiB in + 1 GiB out",
                         "step_frac_of_copy": round(value / copy_gbps, 4)},
        "decode": dec,
        "backward": backward,
        "dispatch_formats": formats,
        "configs": configs,
        "cpu_baseline": cb,
        "cpu_baseline_all_cores": cbp,
        "host_cpu": host_cpu() if cb is not None else None,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
