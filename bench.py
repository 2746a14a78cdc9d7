#!/usr/bin/env python3
"""Throughput of the frame-wise GDN forward on one MI355X, with its roofline and a CPU baseline.

One step = one gdn_forward_framewise call over the whole workload (all frames, all heads) with
the library's schedule for it (fused single pass at this size; --schedule staged times the
three-pass order: products, frame scan, outputs). Inputs are synthetic, seeded and generated on
the device before timing (resident in HBM).

Prints one JSON line. Extra objects:
  roofline      the dominant kernel's algorithmic HBM bytes per launch / its mean launch
                duration, timed with HIP events that the library records around each launch on
                the stream the launch runs on (gdn_set_trace); `traffic` comes from the committed
                rocprofv3 counter summary when it was taken on the current kernel source and
                launch plan, else null.
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload.
  stream        streaming step mode (gdn_step_frame): 4 denoising passes per frame, state
                committed after the last; per-frame latency and frames/s.
  fp8           the same forward from E4M3 Q, K, V with per-frame scales
                (gdn_forward_framewise_fp8): ms per call and its own roofline (Q, K, V at one
                byte per element, O at two).
  tconv         the block-causal temporal conv (gdn_tconv_forward) over the same video at the
                GDN block's width: whole video per call, and per-frame streaming latency.
  attention     frame-causal softmax attention (gdn_attention_framecausal), the hybrid's
                softmax block: the whole 880x81 sequence (TFLOP/s against the bf16 MFMA peak)
                and one 720p frame against the cache of frames 0..f (cost per frame growing with
                f, against the GDN's constant D x D state).
  backward      gdn_backward_framewise over the workload: ms per call, per-kernel ms and the
                call's roofline (Q, K, V, dO read; dQ, dK, dV written).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gdn_720p_60s_bf16.json")
KERNEL_SRC = os.path.join(ROOT, "frame_wise_gated_libgdn_amd", "csrc", "gdn_kernels.hip")
STEP_PROFILE = os.path.join(ROOT, "profiles", "step_kernels_stream_720p_bf16.json")
STEP_SRC = os.path.join(ROOT, "frame_wise_gated_libgdn_amd", "csrc", "gdn_step.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_720p_bench.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t through the HIP runtime that torch already loaded (same soname)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        self.made.append(e.value)
        return e.value

    def record(self, e, stream):
        assert self.rt.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        assert self.rt.hipEventSynchronize(b) == 0
        out = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)

    def close(self):
        for e in self.made:
            self.rt.hipEventDestroy(e)
        self.made = []


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gdn_720p_60s_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time (wall x threads) of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-tconv", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--stream-frames", type=int, default=240)
    ap.add_argument("--step-schedule", default="auto", choices=["auto", "staged"],
                    help="streaming leg: one launch per pass where supported (auto) or three")
    ap.add_argument("--schedule", default="auto", choices=["auto", "staged", "fused"],
                    help="forward schedule (auto: the library's choice)")
    ap.add_argument("--copy-calib-gib", type=float, default=0.0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--placement-sweep", type=int, default=0,
                    help="only the 720p forward at this many output placements (for counter runs)")
    ap.add_argument("--stream-only", action="store_true",
                    help="only the streaming step leg (for profiling its kernels); prints its JSON")
    return ap.parse_args()


def source_sha(path=KERNEL_SRC):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def step_profile():
    """Average duration (us) of each step-mode kernel from the committed rocprofv3 kernel trace
    of the streaming workload, if it was taken on the current step-kernel source; else None."""
    try:
        with open(STEP_PROFILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha(STEP_SRC):
        return None
    return {k: v["avg_us"] for k, v in t.get("kernels", {}).items()}


def traffic_for(kernel, workload, plan):
    """Counter-derived HBM bytes per launch (GB), if measured on the current kernel source with
    the same launch plan."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha() or t.get("workload") != workload \
            or t.get("plan") != plan:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else round(k["hbm_gb_per_launch"], 3)


def counters_for(key=None):
    """Committed rocprofv3 counters of one kernel of the bench's legs (HBM bytes, L2 hit rate,
    MFMA busy fraction, clock), or of all of them when key is None; an entry is None when its
    kernel's source changed since the counters were taken."""
    try:
        with open(COUNTERS_FILE) as fh:
            t = json.load(fh)["kernels"]
    except (OSError, ValueError, KeyError):
        return None
    csrc = os.path.join(ROOT, "frame_wise_gated_libgdn_amd", "csrc")

    def entry(e):
        if e.get("source_sha256") != source_sha(os.path.join(csrc, e["source"])):
            return None
        return {k_: e[k_] for k_ in ("avg_us", "hbm_read_gb", "hbm_write_gb", "l2_hit",
                                     "mfma_busy", "mfma_busy_at_2400mhz", "bf16_mfma_tflops",
                                     "clock_ghz")}
    if key is not None:
        return entry(t[key]) if key in t else None
    return {k_: entry(e) for k_, e in t.items()}


def copy_calibration(gib):
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds):
    """The fp64 oracle (plain C loops, OpenMP over independent heads) on a bounded sample of
    the workload, on every core this process may run on; plus one head on one thread, and a
    sample of the streaming protocol (whole-state passes of every head from the oracle's own
    committed state)."""
    import numpy as np
    import gdn_synth
    import oracle
    # the oracle is parallel over independent (b, h) only, so more threads than heads idle
    avail = len(os.sched_getaffinity(0))
    nthreads = max(1, min(avail, w.B * w.H))
    heads = list(range(w.H))

    def run(nf, hs, threads):
        (q, k, v), _ = gdn_synth.qkv_cpu(w, heads=hs, frames=range(nf))
        g, b = gdn_synth.gates_cpu(w, heads=hs, frames=range(nf))
        t = time.perf_counter()
        oracle.forward(q, k, v, g, b, use_delta=w.use_delta, nthreads=threads)
        return time.perf_counter() - t

    t1 = run(1, heads, nthreads)
    nf = int(max(1, min(16, w.F, round(seconds / max(t1 * nthreads, 1e-6)))))
    log("cpu baseline: 1 frame took %.2f s; timing %d frames on %d threads" % (t1, nf, nthreads))
    t = run(nf, heads, nthreads) if nf > 1 else t1
    tokens = w.B * nf * w.S
    # one head on one thread
    nf1 = 2
    t_one = run(nf1, [0], 1)
    # the streaming protocol (one frame, 4 passes, commit after the last) on a sample of frames
    ws = gdn_synth.WORKLOADS["stream_720p_bf16"]
    sf = 2
    M = np.zeros((ws.B, ws.H, ws.D, ws.D))
    ts = 0.0
    for f in range(sf):
        for p in range(ws.passes):
            (q, k, v), _ = gdn_synth.qkv_cpu(ws, frames=[f], pass_=p)
            g, b = gdn_synth.gates_cpu(ws, frames=[f], pass_=p)
            t0 = time.perf_counter()
            _, Mn = oracle.step(q, k, v, g[..., 0], b[..., 0], M, commit=True, nthreads=nthreads)
            ts += time.perf_counter() - t0
        M = Mn
    return {"value": round(tokens / t, 1), "unit": "tokens/s", "cores": nthreads,
            "cores_available": avail,
            "kind": "oracle", "seconds": round(t, 2), "cpu_model": cpu_model(),
            "sample": "all %d heads of batch 0, frames 0-%d of %s (S=%d, D=%d): fp64 oracle, "
                      "OpenMP over heads" % (w.H, nf - 1, w.name, w.S, w.D),
            "single_thread_one_head": {"tokens_per_s": round(w.B * nf1 * w.S / t_one, 1),
                                       "seconds": round(t_one, 2),
                                       "sample": "head 0, frames 0-%d, 1 thread" % (nf1 - 1)},
            "stream": {"frames_per_s": round(sf / ts, 3), "seconds": round(ts, 2),
                       "sample": "%s: frames 0-%d x %d passes, all %d heads, %d threads"
                                 % (ws.name, sf - 1, ws.passes, ws.H, nthreads)}}


def stream_mode(dev, nframes, ev, stream, schedule="auto"):
    """Streaming step mode: per frame 4 passes from the same incoming state, commit on the last.
    The timed loop issues prepared gdn_step_frame calls (arguments marshalled once, as a serving
    loop holding its buffers would), so that it measures the library rather than the binding's
    per-call checks; the plain binding call is timed beside it."""
    import time
    import numpy as np
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    w = gdn_synth.WORKLOADS["stream_720p_bf16"]
    nframes = min(nframes, w.F)
    gen = gdn_synth.TorchGen(dev)
    passes = []
    for p in range(w.passes):
        q, k, v = gdn_synth.qkv_torch(w, dev, frames=(0, nframes), pass_=p, gen=gen)
        g, b = gdn_synth.gates_torch(w, dev, pass_=p)
        # per-frame gates as contiguous [B, H] slices
        gf, bf = g.permute(2, 0, 1).contiguous(), b.permute(2, 0, 1).contiguous()
        passes.append((q, k, v, [gf[f] for f in range(nframes)], [bf[f] for f in range(nframes)]))
    state = torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev)
    wsz = gdn.workspace_size(gdn.Problem(w.B, w.H, w.D, w.S, 1, gdn.GDN_BF16, 1, 0.0,
                                         0, 0, w.D, 0, 0, w.D, gdn.SCHEDULES[schedule]), True)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

    def args(f, p):
        sl = slice(f * w.S, (f + 1) * w.S)
        q, k, v, g, b = passes[p]
        last = p == w.passes - 1
        return (q[:, :, sl], k[:, :, sl], v[:, :, sl], g[f], b[f], state), \
            dict(commit=last, out=o, state_out=state if last else None, workspace=ws,
                 schedule=schedule)

    calls = []
    for f in range(nframes):
        row = []
        for p in range(w.passes):
            a, kw = args(f, p)
            row.append(gdn.prepare_step_frame(*a, **kw))
        calls.append(row)

    def timed(frame_fn):
        for f in range(min(3, nframes)):  # warm-up
            frame_fn(f)
        state.zero_()
        torch.cuda.synchronize()
        marks = [ev.new() for _ in range(nframes + 1)]
        t0 = time.perf_counter()
        ev.record(marks[0], stream)
        for f in range(nframes):
            frame_fn(f)
            ev.record(marks[f + 1], stream)
        host = time.perf_counter() - t0
        torch.cuda.synchronize()
        lat = np.array([ev.ms(marks[f], marks[f + 1]) for f in range(nframes)])
        return lat, ev.ms(marks[0], marks[-1]), host

    def prepared(f):
        for c in calls[f]:
            c()

    def binding(f):
        for p in range(w.passes):
            a, kw = args(f, p)
            gdn.step_frame(*a, **kw)

    lat, total, host = timed(prepared)
    blat, btotal, bhost = timed(binding)
    # per-kernel split of one pass, from the launch trace, over a few extra frames (untimed above)
    kus = {}
    for f in range(min(8, nframes)):
        a, kw = args(f, 0)
        tr = [ev.new() for _ in range(6)]
        gdn.set_trace(tr)
        gdn.step_frame(*a, **kw)
        plan = gdn.read_trace()
        gdn.set_trace(None)
        for j, (kname, _, _) in enumerate(plan):
            kus.setdefault(kname, []).append(ev.ms(tr[2 * j], tr[2 * j + 1]) * 1e3)
    npass = nframes * w.passes
    return {"workload": w.name, "frames": nframes, "passes_per_frame": w.passes,
            "schedule": schedule, "launches_per_pass": len(kus),
            "frame_latency_ms": {"median": round(float(np.median(lat)), 4),
                                 "p90": round(float(np.percentile(lat, 90)), 4),
                                 "max": round(float(lat.max()), 4)},
            "frames_per_s": round(nframes / (total / 1e3), 1),
            "pass_us_median": round(float(np.median(lat)) * 1e3 / w.passes, 2),
            # host time to enqueue a pass in the timed loop: below the pass time, the GPU is the
            # bound
            "host_us_per_pass": round(host * 1e6 / npass, 2),
            # the same protocol through the checking binding call step_frame on every pass
            "binding": {"pass_us_median": round(float(np.median(blat)) * 1e3 / w.passes, 2),
                        "host_us_per_pass": round(bhost * 1e6 / npass, 2)},
            # each launch bracketed by its own events (the events add gaps between launches, so
            # these sum to more than a pass), and the rocprofv3 kernel averages of the same
            # workload from the committed summary (null when taken on other kernel source)
            "pass_kernel_us_traced": {k_: round(float(np.median(v_)), 2) for k_, v_ in kus.items()},
            "pass_kernel_us_rocprof": step_profile(),
            "same_bytes_torch_us": round(pass_bytes_reference(dev, w.B * w.H * w.S * w.D), 2)}


def backward_mode(w, dev, steps, ev, stream):
    """Training direction: one gdn_backward_framewise call over the whole workload (forward
    states recomputed inside), for upstream gradients dO of the output's shape."""
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    gen = gdn_synth.TorchGen(dev)
    q, k, v = gdn_synth.qkv_torch(w, dev, gen=gen)
    g, b = gdn_synth.gates_torch(w, dev)
    d_o = torch.empty_like(q)
    for bb in range(w.B):
        for hh in range(w.H):   # seeded like Q, from another seed
            gen.fill_normal(d_o[bb, hh], w.seed + 1000, gdn_synth.TID_Q, bb, hh, 0, w.S, w.D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    p = gdn.Problem(w.B, w.H, w.D, w.S, w.F, gdn.GDN_BF16, int(w.use_delta), 0.0, *q.stride()[:3],
                    *d_o.stride()[:3])
    ws = torch.empty(gdn.workspace_size(p, 2), dtype=torch.uint8, device=dev)

    def call():
        return gdn.backward_framewise(q, k, v, g, b, d_o, use_delta=w.use_delta, dq=dq, dk=dk,
                                      dv=dv, workspace=ws, stream=stream)

    probe = [ev.new() for _ in range(2 * 16)]
    gdn.set_trace(probe)
    call()
    plan = gdn.read_trace()
    gdn.set_trace(None)
    call()
    torch.cuda.synchronize()
    nl = len(plan)
    trace = [[ev.new() for _ in range(2 * nl)] for _ in range(steps)]
    t0, t1 = ev.new(), ev.new()
    sh = stream.cuda_stream
    ev.record(t0, sh)
    for i in range(steps):
        gdn.set_trace(trace[i])
        call()
    gdn.set_trace(None)
    ev.record(t1, sh)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    kms = {}
    for i in range(steps):
        for j, (kname, _, _) in enumerate(plan):
            kms[kname] = kms.get(kname, 0.0) + ev.ms(trace[i][2 * j], trace[i][2 * j + 1]) / steps
    esz = w.elem_bytes()
    bytes_alg = 7 * w.B * w.H * w.F * w.S * w.D * esz   # Q, K, V, dO read; dQ, dK, dV written
    flops_alg = (10 if w.use_delta else 6) * w.B * w.H * w.F * w.S * w.D * w.D
    t_roof = max(bytes_alg / (HBM_PEAK_GBS * 1e9), flops_alg / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    bwd_ms = kms.get("bwd", 0.0)
    bwd_bytes = 4 * w.B * w.H * w.F * w.S * w.D * esz   # per-frame gradient kernel: K, V, dK, dV
    qdo_ms = kms.get("bwd_qdo", 0.0)
    qdo_bytes = 3 * w.B * w.H * w.F * w.S * w.D * esz   # pass over Q and dO: Q, dO, dQ
    del ws

    # training with saved states: the fused forward that keeps the states and Ghat records,
    # then the backward from them (no forward recompute)
    o = torch.empty_like(q)
    pf = gdn.Problem(w.B, w.H, w.D, w.S, w.F, gdn.GDN_BF16, int(w.use_delta), 0.0, *q.stride()[:3],
                     *o.stride()[:3], gdn.SCHEDULES["fused"])
    saved = torch.empty(gdn.saved_size(pf), dtype=torch.uint8, device=dev)
    wsf = torch.empty(gdn.workspace_size(pf, 0), dtype=torch.uint8, device=dev)
    ws3 = torch.empty(gdn.workspace_size(p, 3), dtype=torch.uint8, device=dev)

    def fwd_save():
        gdn.forward_framewise_save(q, k, v, g, b, use_delta=w.use_delta, out=o, return_state=False,
                                   saved=saved, workspace=wsf, stream=stream)

    def bwd_saved():
        gdn.backward_framewise(q, k, v, g, b, d_o, use_delta=w.use_delta, dq=dq, dk=dk, dv=dv,
                               saved=saved, workspace=ws3, stream=stream)

    def timed(f):
        f()
        torch.cuda.synchronize()
        a, z = ev.new(), ev.new()
        ev.record(a, sh)
        for _ in range(steps):
            f()
        ev.record(z, sh)
        torch.cuda.synchronize()
        return ev.ms(a, z) / steps

    fs_ms = timed(fwd_save)
    bs_ms = timed(bwd_saved)
    saved_gb = saved.numel() / 1e9
    del q, k, v, d_o, dq, dk, dv, o, saved, wsf, ws3
    torch.cuda.empty_cache()
    ceil_1r = {"kind": CEILING_KINDS[1], "gb_s": round(streaming_ceiling(dev, 1), 1)}
    ceil_2r = {"kind": CEILING_KINDS[2], "gb_s": round(streaming_ceiling(dev, 2), 1)}
    return {"workload": w.name, "ms_per_call": round(ms, 4),
            "from_saved_states": {"forward_save_ms": round(fs_ms, 4), "saved_gb": round(saved_gb, 3),
                                  "backward_ms": round(bs_ms, 4),
                                  "backward_frac_of_roofline": round(t_roof / bs_ms, 4)},
            "tokens_per_s": round(w.B * w.F * w.S / (ms * 1e-3), 1),
            "launches": [k_ for k_, _, _ in plan],
            "kernel_ms_per_call": {k_: round(x, 4) for k_, x in kms.items()},
            "call": {"bytes_alg_gb": round(bytes_alg / 1e9, 3), "t_roof_ms": round(t_roof, 4),
                     "frac_of_roofline": round(t_roof / ms, 4),
                     "achieved_gb_s": round(bytes_alg / (ms * 1e-3) / 1e9, 1)},
            "bwd_kernel": kernel_vs_ceiling(bwd_bytes, bwd_ms, "bwd", ceil_1r),
            "qdo_kernel": kernel_vs_ceiling(qdo_bytes, qdo_ms, "qdo", ceil_2r)}


def kernel_vs_ceiling(alg_bytes, ms, key, ceiling):
    """A backward kernel's algorithmic rate against the HBM peak; its measured HBM traffic (the
    committed counters, when they were taken on the current source) per this run's duration,
    against the torch streaming kernel with its mix of reads and writes."""
    if not ms:
        return None
    c = counters_for(key)
    hbm = c["hbm_read_gb"] + c["hbm_write_gb"] if c else None
    out = {"achieved_gb_s": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
           "frac": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "hbm_gb_per_launch": round(hbm, 3) if hbm else None,
           "hbm_gb_s": round(hbm / (ms * 1e-3), 1) if hbm else None,
           "ceiling": ceiling}
    out["frac_of_ceiling"] = round(hbm / (ms * 1e-3) / ceiling["gb_s"], 4) if hbm else None
    return out


def fp8_mode(dev, steps, warmup, ev, stream):
    """The 720p forward from E4M3 Q, K, V (one scale per (b, h, f) and tensor), bf16 output."""
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    w = gdn_synth.WORKLOADS["gdn_720p_60s_fp8"]
    (q, k, v), (sq, sk, sv) = gdn_synth.qkv_fp8_torch(w, dev)
    g, b = gdn_synth.gates_torch(w, dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    p = gdn.Problem(w.B, w.H, w.D, w.S, w.F, gdn.GDN_FP8_E4M3, int(w.use_delta), 0.0,
                    *q.stride()[:3], *o.stride()[:3])
    ws = torch.empty(gdn.workspace_size(p, False), dtype=torch.uint8, device=dev)

    def call():
        gdn.forward_framewise_fp8(q, k, v, sq, sk, sv, g, b, use_delta=w.use_delta, out=o,
                                  state_out=st, workspace=ws, stream=stream)

    probe = [ev.new() for _ in range(2 * 16)]
    gdn.set_trace(probe)
    call()
    plan = gdn.read_trace()
    gdn.set_trace(None)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    nl = len(plan)
    trace = [[ev.new() for _ in range(2 * nl)] for _ in range(steps)]
    t0, t1 = ev.new(), ev.new()
    sh = stream.cuda_stream
    ev.record(t0, sh)
    for i in range(steps):
        gdn.set_trace(trace[i])
        call()
    gdn.set_trace(None)
    ev.record(t1, sh)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    kms = {}
    for i in range(steps):
        for j, (kname, _, _) in enumerate(plan):
            kms[kname] = kms.get(kname, 0.0) + ev.ms(trace[i][2 * j], trace[i][2 * j + 1]) / steps
    n = w.B * w.H * w.F * w.S * w.D
    bytes_alg = 3 * n * 1 + n * 2      # E4M3 Q, K, V read; bf16 O written (scales, gates ~0)
    flops_alg = (6 if w.use_delta else 4) * n * w.D
    t_roof = max(bytes_alg / (HBM_PEAK_GBS * 1e9), flops_alg / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    fms = kms.get("fused", 0.0)
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    c = counters_for("fused_e4m3")
    hbm = c["hbm_read_gb"] + c["hbm_write_gb"] if c else None
    return {"workload": w.name, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(w.B * w.F * w.S / (ms * 1e-3), 1),
            "launches": [k_ for k_, _, _ in plan],
            "kernel_ms_per_call": {k_: round(x, 4) for k_, x in kms.items()},
            "call": {"bytes_alg_gb": round(bytes_alg / 1e9, 3), "t_roof_ms": round(t_roof, 4),
                     "frac_of_roofline": round(t_roof / ms, 4),
                     "achieved_gb_s": round(bytes_alg / (ms * 1e-3) / 1e9, 1)},
            "fused_kernel": {"achieved_gb_s": round(bytes_alg / (fms * 1e-3) / 1e9, 1) if fms else None,
                             "frac": round(bytes_alg / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if fms else None,
                             # the kernel's measured HBM traffic (committed counters) per this
                             # run's duration
                             "hbm_gb_per_launch": round(hbm, 3) if hbm else None,
                             "hbm_gb_s": round(hbm / (fms * 1e-3), 1) if fms and hbm else None}}


def tconv_mode(dev, steps, warmup, ev, stream, stream_frames=240):
    """Block-causal temporal conv at the GDN block's width (tconv_720p_60s_bf16): the whole
    video in one call (training form), then frame-by-frame streaming from the cache (one block
    per call, cache updated in place)."""
    import numpy as np
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    w = gdn_synth.TCONV_WORKLOADS["tconv_720p_60s_bf16"]
    x = gdn_synth.tconv_x_torch(w, dev)
    taps, bias = gdn_synth.tconv_weights(w)
    wt, bt = torch.from_numpy(taps).to(dev), torch.from_numpy(bias).to(dev)
    y = torch.empty_like(x)
    cache = torch.empty((w.B, w.S, w.C), dtype=x.dtype, device=dev)
    sh = stream.cuda_stream

    def whole():
        gdn.temporal_conv(x, wt, bt, None, block_frames=w.block_frames, out=y, cache_out=cache,
                          stream=stream)

    for _ in range(warmup + 1):
        whole()
    torch.cuda.synchronize()
    trace = [[ev.new(), ev.new()] for _ in range(steps)]
    t0, t1 = ev.new(), ev.new()
    ev.record(t0, sh)
    for i in range(steps):
        gdn.set_trace(trace[i])
        whole()
    gdn.set_trace(None)
    ev.record(t1, sh)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    kms = sum(ev.ms(a, b) for a, b in trace) / steps
    n = w.B * w.T * w.S * w.C
    bytes_alg = 2 * n * 2                      # x read, y written (bf16)
    # streaming: one frame per call from the previous frame's cache
    nf = min(stream_frames, w.T)
    yf = torch.empty((w.B, 1, w.S, w.C), dtype=x.dtype, device=dev)
    c = torch.zeros_like(cache)
    for f in range(3):
        gdn.temporal_conv(x[:, f:f + 1], wt, bt, c, block_frames=1, out=yf, cache_out=c, stream=stream)
    torch.cuda.synchronize()
    # frame by frame through prepared calls (arguments marshalled once, as a streaming loop
    # holding its buffers would), one event between frames
    calls = [gdn.prepare_temporal_conv(x[:, f:f + 1], wt, bt, c, block_frames=1, out=yf, cache_out=c,
                                       stream=stream) for f in range(nf)]
    marks = [ev.new() for _ in range(nf + 1)]
    ev.record(marks[0], sh)
    for f in range(nf):
        calls[f]()
        ev.record(marks[f + 1], sh)
    torch.cuda.synchronize()
    lat = np.array([ev.ms(marks[f], marks[f + 1]) * 1e3 for f in range(nf)])
    # the same through the checking binding call, each launch bracketed by its own events
    evs = [(ev.new(), ev.new()) for _ in range(nf)]
    kev = [[ev.new(), ev.new()] for _ in range(nf)]
    for f in range(nf):
        ev.record(evs[f][0], sh)
        gdn.set_trace(kev[f])
        gdn.temporal_conv(x[:, f:f + 1], wt, bt, c, block_frames=1, out=yf, cache_out=c, stream=stream)
        ev.record(evs[f][1], sh)
    gdn.set_trace(None)
    torch.cuda.synchronize()
    blat = np.array([ev.ms(a, b) * 1e3 for a, b in evs])      # includes the host's launch work
    klat = np.array([ev.ms(a, b) * 1e3 for a, b in kev])      # the launch alone
    step_bytes = 4 * w.B * w.S * w.C * 2       # x, cache_in read; y, cache_out written
    del x, y
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms_per_call": round(ms, 4), "kernel_ms": round(kms, 4),
            "frames_per_s": round(w.T / (ms * 1e-3), 1),
            "bytes_alg_gb": round(bytes_alg / 1e9, 3),
            "achieved_gb_s": round(bytes_alg / (kms * 1e-3) / 1e9, 1),
            "frac": round(bytes_alg / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stream": {"frames": nf, "us_per_frame_median": round(float(np.median(lat)), 2),
                       "us_per_frame_p90": round(float(np.percentile(lat, 90)), 2),
                       "binding_us_per_frame_median": round(float(np.median(blat)), 2),
                       "kernel_us_median": round(float(np.median(klat)), 2),
                       "kernel_gb_s": round(step_bytes / (float(np.median(klat)) * 1e-6) / 1e9, 1),
                       "bytes_per_frame_mb": round(step_bytes / 1e6, 2),
                       "floor_us": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}}


def attention_mode(dev, steps, warmup, ev, stream):
    """Frame-causal softmax attention (the hybrid's softmax block) at the pages' frame shapes:
    the whole 880x81 sequence, and one 720p frame against the key/value cache of frames 0..f,
    the per-frame cost that the GDN's constant state replaces."""
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    sh = stream.cuda_stream

    def timed(fn, reps):
        """ms per call: the sum of the call's launches (one, or two with key splits)."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        tr = [[ev.new() for _ in range(4)] for _ in range(reps)]
        nl = 1
        for i in range(reps):
            gdn.set_trace(tr[i])
            fn()
            nl = len(gdn.read_trace())
        gdn.set_trace(None)
        torch.cuda.synchronize()
        return sum(sum(ev.ms(t[2 * j], t[2 * j + 1]) for j in range(nl)) for t in tr) / reps, nl

    out = {}
    w = gdn_synth.WORKLOADS["gdn_880x81_bf16"]
    q, k, v = gdn_synth.qkv_torch(w, dev)
    o = torch.empty_like(q)
    ms, _ = timed(lambda: gdn.attention_framecausal(q, k, v, tokens_per_frame=w.S, out=o, stream=stream),
                  steps)
    flops = 4 * w.D * w.S * w.S * w.F * (w.F + 1) // 2 * w.B * w.H
    out["whole_880x81"] = {"workload": w.name, "kernel_ms": round(ms, 4),
                           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                           "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                           "flops_alg_tf": round(flops / 1e12, 3)}
    del q, k, v, o
    torch.cuda.empty_cache()
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    S = w.S
    q, k, v = gdn_synth.qkv_torch(w, dev)
    o = torch.empty((w.B, w.H, S, w.D), dtype=torch.bfloat16, device=dev)
    per = []
    for f in (60, 240, w.F - 1):
        n = (f + 1) * S
        qf, kf, vf = q[:, :, f * S:(f + 1) * S], k[:, :, :n], v[:, :, :n]
        # a workspace lets the call split each query block's keys over more workgroups
        nb = gdn.attention_workspace_size(gdn.attention_problem(qf, kf, o, S, f))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        ms, nl = timed(lambda: gdn.attention_framecausal(qf, kf, vf, tokens_per_frame=S, q_frame0=f, out=o,
                                                         workspace=ws, stream=stream),
                       max(1, min(steps, 5)))
        flops = 4 * w.D * S * n * w.B * w.H
        per.append({"frame": f, "kernel_ms": round(ms, 3), "launches": nl,
                    "workspace_mb": round(nb / 1e6, 1),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "kv_cache_gb": round(2 * n * w.D * 2 * w.B * w.H / 1e9, 2)})
        del ws
    out["stream_720p_frame"] = {"workload": w.name, "per_frame": per,
                                "gdn_state_mb": round(w.B * w.H * w.D * w.D * 4 / 1e6, 2)}
    del q, k, v, o
    torch.cuda.empty_cache()
    return out


def placement_sweep(dev, count, reps=3):
    """The 720p forward with the same Q, K, V and a new output buffer for each of `count`
    placements (every earlier buffer kept, so each lands on fresh pages further away in HBM):
    ms per call at each placement, for counter runs that compare them (dispatches in order)."""
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    w = gdn_synth.WORKLOADS["gdn_720p_60s_bf16"]
    q, k, v = gdn_synth.qkv_torch(w, dev)
    g, b = gdn_synth.gates_torch(w, dev)
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    p = gdn.Problem(w.B, w.H, w.D, w.S, w.F, gdn.GDN_BF16, int(w.use_delta), 0.0,
                    *q.stride()[:3], *q.stride()[:3])
    ws = torch.empty(gdn.workspace_size(p, False), dtype=torch.uint8, device=dev)
    outs, rows = [], []
    base = q.data_ptr()
    for i in range(count):
        o = torch.empty_like(q)
        outs.append(o)
        gdn.forward_framewise(q, k, v, g, b, out=o, state_out=st, workspace=ws)   # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gdn.forward_framewise(q, k, v, g, b, out=o, state_out=st, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        rows.append({"placement": i, "o_offset_gb": round((o.data_ptr() - base) / 1e9, 2),
                     "ms": round(e0.elapsed_time(e1) / reps, 4)})
        log("placement %d: O at +%.2f GB from Q, %.3f ms" % (i, rows[-1]["o_offset_gb"], rows[-1]["ms"]))
    return {"workload": w.name, "reps_per_placement": reps, "dispatches_per_placement": reps + 1,
            "placements": rows}


CEILING_KINDS = {
    1: "torch bf16 copy y = a: 1 tensor read, 1 written, 4 GiB each",
    2: "torch bf16 add y = a + b: 2 tensors read, 1 written, 4 GiB each",
    3: "torch bf16 addcmul y = a + b * c: 3 tensors read, 1 written, 4 GiB each",
}


def streaming_ceiling(dev, nread=3, gib=4.0, reps=10):
    """Bandwidth of a plain torch streaming kernel that reads `nread` tensors and writes one
    (one elementwise kernel): the reference for a kernel with the same mix of traffic (the fused
    forward reads three and writes one; the backward's Q/dO pass two and one; its gradient
    kernel K, V and dK, dV, one to one)."""
    import torch
    n = int(gib * (1 << 30)) // 2
    xs = [torch.empty(n, dtype=torch.bfloat16, device=dev).normal_() for _ in range(nread)]
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)

    def f():
        if nread == 1:
            y.copy_(xs[0])
        elif nread == 2:
            torch.add(xs[0], xs[1], out=y)
        else:
            torch.addcmul(xs[0], xs[1], xs[2], out=y)

    f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del xs, y
    torch.cuda.empty_cache()
    return (nread + 1) * n * 2 / (ms * 1e-3) / 1e9


def pass_bytes_reference(dev, n, reps=200):
    """Time of one torch elementwise kernel that moves a step pass's algorithmic bytes (three
    bf16 tensors of n elements read, one written), launched back to back: what streaming the
    same bytes with no dependency between them costs at this size."""
    import torch
    xs = [torch.empty(n, dtype=torch.bfloat16, device=dev).normal_() for _ in range(3)]
    y = torch.empty(n, dtype=torch.bfloat16, device=dev)
    for _ in range(10):
        torch.addcmul(xs[0], xs[1], xs[2], out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.addcmul(xs[0], xs[1], xs[2], out=y)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    del xs, y
    return us


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(asked for --gpus %d, WORLD_SIZE=%d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    import frame_wise_gated_libgdn_amd as gdn
    import gdn_synth
    if args.copy_calib_gib > 0:
        copy_calibration(args.copy_calib_gib)
        return
    gdn.load()
    if args.placement_sweep > 0:
        print(json.dumps({"placement_sweep": placement_sweep(torch.device("cuda:0"),
                                                             args.placement_sweep)}), flush=True)
        return
    if args.stream_only:
        ev = HipEvents()
        print(json.dumps({"stream": stream_mode(torch.device("cuda:0"), args.stream_frames, ev,
                                                torch.cuda.current_stream().cuda_stream,
                                                args.step_schedule)}), flush=True)
        ev.close()
        return
    w = gdn_synth.WORKLOADS[args.workload]
    assert not w.step_mode, "the forward bench needs a forward workload"
    dev = torch.device("cuda:0")
    log("generating %s inputs on the device" % w.name)
    t = time.perf_counter()
    q, k, v = gdn_synth.qkv_torch(w, dev)
    g, b = gdn_synth.gates_torch(w, dev)
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.perf_counter() - t))
    o = torch.empty_like(q)
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=dev)
    p = gdn.Problem(w.B, w.H, w.D, w.S, w.F, gdn.GDN_BF16 if w.dtype == "bf16" else gdn.GDN_F32,
                    int(w.use_delta), 0.0, *q.stride()[:3], *o.stride()[:3],
                    gdn.SCHEDULES[args.schedule])
    ws = torch.empty(gdn.workspace_size(p, False), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call():
        gdn.forward_framewise(q, k, v, g, b, use_delta=w.use_delta, out=o, state_out=st,
                              workspace=ws, stream=stream, schedule=args.schedule)

    ev = HipEvents()
    # one traced warm-up call gives the launch plan (kernel, stream, units of each launch)
    probe = [ev.new() for _ in range(2 * 256)]
    gdn.set_trace(probe)
    call()
    plan = gdn.read_trace()
    gdn.set_trace(None)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log("warm-up done (%d steps); %d launches per step: %s" % (
        args.warmup, len(plan), " ".join("%s%s:%d" % (k_[0], "'" if s_ else "", u)
                                          for k_, s_, u in plan)))

    nl = len(plan)
    trace = [[ev.new() for _ in range(2 * nl)] for _ in range(args.steps)]
    t0, t1 = ev.new(), ev.new()
    torch.cuda.synchronize()
    ev.record(t0, sh)
    for i in range(args.steps):
        gdn.set_trace(trace[i])
        call()
    gdn.set_trace(None)
    ev.record(t1, sh)
    torch.cuda.synchronize()
    total_ms = ev.ms(t0, t1)
    ms = total_ms / args.steps
    esz = w.elem_bytes()
    # algorithmic HBM bytes per (b, h, frame) item: a products item streams K and V (gram) or
    # Q and O (outputs); a fused item streams all four
    unit_bytes = {"products": 2 * w.S * w.D * esz, "fused": 4 * w.S * w.D * esz}
    per = {}                                    # kernel -> [launches, ms, units]
    for i in range(args.steps):
        for j, (kname, _, units) in enumerate(plan):
            acc = per.setdefault(kname, [0, 0.0, 0])
            acc[0] += 1
            acc[1] += ev.ms(trace[i][2 * j], trace[i][2 * j + 1])
            acc[2] += units
    kms = {k_: a[1] / args.steps for k_, a in per.items()}
    # per call: from the first launch's start event to the last launch's end event
    calls = sorted(ev.ms(trace[i][0], trace[i][2 * nl - 1]) for i in range(args.steps))
    call_median = calls[len(calls) // 2] if len(calls) % 2 else 0.5 * (calls[len(calls) // 2 - 1] + calls[len(calls) // 2])
    log("timed %d steps: %.3f ms/step (median %.3f, min %.3f); summed launch ms per step %s" % (
        args.steps, ms, call_median, calls[0], {k_: round(x, 3) for k_, x in kms.items()}))

    tokens = w.B * w.F * w.S
    bytes_alg = 4 * w.B * w.H * w.F * w.S * w.D * esz          # Q, K, V read + O written
    flops_alg = (6 if w.use_delta else 4) * w.B * w.H * w.F * w.S * w.D * w.D
    dom = max((k_ for k_ in per if k_ in unit_bytes), key=lambda k_: per[k_][1])
    n_l, ms_l, units_l = per[dom]
    launch_ms = ms_l / n_l
    launch_bytes = units_l * unit_bytes[dom] / n_l
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
    plan_key = [[k_, s_, u] for k_, s_, u in plan]
    t_roof_ms = max(bytes_alg / (HBM_PEAK_GBS * 1e9), flops_alg / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    result = {
        "metric": "GDN tokens/sec at 961x3520-token 720p shape; % of HBM/MFMA roofline",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_call_median": round(call_median, 4),
        "ms_per_call_min": round(calls[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.D,
                   "tokens_per_frame": w.S, "frames": w.F, "tokens": tokens,
                   "use_delta": w.use_delta, "layout": "head-major [B,H,T,D]",
                   "state": "fp32", "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm", "kernel": dom + "_kernel",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(dom + "_kernel", w.name, plan_key),
            "traffic_unit": "GB per launch",
            # MFMA busy fraction and L2 hit rate of the same kernel from committed counters
            "mfma_busy": (counters_for("fused_bf16") or {}).get("mfma_busy"),
            "l2_hit": (counters_for("fused_bf16") or {}).get("l2_hit"),
            "algorithmic_gb_per_launch": round(launch_bytes / 1e9, 4),
            "launch_ms": round(launch_ms, 4),
            "launches_per_step": {k_: a[0] // args.steps for k_, a in per.items()},
            "plan": plan_key,
            "kernel_ms_per_step": {k_: round(x, 4) for k_, x in kms.items()},
            "schedule": args.schedule,
            "call": {"bytes_alg_gb": round(bytes_alg / 1e9, 3),
                     "flops_alg_tf": round(flops_alg / 1e12, 4),
                     "t_roof_ms": round(t_roof_ms, 4),
                     "frac_of_roofline": round(t_roof_ms / ms, 4),
                     "achieved_gb_s": round(bytes_alg / (ms * 1e-3) / 1e9, 1),
                     "achieved_tflops": round(flops_alg / (ms * 1e-3) / 1e12, 2)},
        },
    }
    ev.close()
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    ceil = streaming_ceiling(dev, 3)
    result["roofline"]["streaming_ceiling"] = {
        "kind": CEILING_KINDS[3],
        "gb_s": round(ceil, 1), "frac_of_ceiling": round(achieved / ceil, 4)}
    log("streaming ceiling (torch addcmul): %.0f GB/s" % ceil)
    if not args.no_stream:
        ev2 = HipEvents()
        log("streaming step mode: %d frames x 4 passes" % args.stream_frames)
        result["stream"] = stream_mode(dev, args.stream_frames, ev2, sh, args.step_schedule)
        ev2.close()
        log("stream done: %s" % result["stream"]["frame_latency_ms"])
    if not args.no_fp8 and w.name == "gdn_720p_60s_bf16":
        ev4 = HipEvents()
        log("fp8 inputs: %d calls" % args.steps)
        result["fp8"] = fp8_mode(dev, args.steps, args.warmup, ev4, torch.cuda.current_stream())
        ev4.close()
        torch.cuda.empty_cache()
        log("fp8 done: %.3f ms/call" % result["fp8"]["ms_per_call"])
    if not args.no_tconv and w.name == "gdn_720p_60s_bf16":
        ev5 = HipEvents()
        log("temporal conv: %d calls" % args.steps)
        result["tconv"] = tconv_mode(dev, args.steps, args.warmup, ev5, torch.cuda.current_stream())
        ev5.close()
        torch.cuda.empty_cache()
        log("temporal conv done: %.3f ms/call" % result["tconv"]["ms_per_call"])
    if not args.no_attention and w.name == "gdn_720p_60s_bf16":
        ev6 = HipEvents()
        log("softmax attention")
        result["attention"] = attention_mode(dev, args.steps, min(args.warmup, 1), ev6,
                                             torch.cuda.current_stream())
        ev6.close()
        torch.cuda.empty_cache()
        log("attention done: %s" % result["attention"]["whole_880x81"])
    if not args.no_backward and w.dtype == "bf16" and w.D in (64, 128):
        ev3 = HipEvents()
        log("backward: %d calls" % args.backward_steps)
        result["backward"] = backward_mode(w, dev, args.backward_steps, ev3, torch.cuda.current_stream())
        ev3.close()
        torch.cuda.empty_cache()
        log("backward done: %.3f ms/call; from saved states %.3f ms/call (saving forward %.3f ms)" % (
            result["backward"]["ms_per_call"], result["backward"]["from_saved_states"]["backward_ms"],
            result["backward"]["from_saved_states"]["forward_save_ms"]))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    if w.name == "gdn_720p_60s_bf16":
        # per-kernel counters of every leg (rocprofv3 runs of this script, committed summary)
        result["counters"] = counters_for()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
