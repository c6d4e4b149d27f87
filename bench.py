#!/usr/bin/env python3
"""WBMM benchmark on one MI355X: the layer's training step (forward + backward) at w = 14.

A step is one pass of the whole hot path over one synthetic batch of the training workload
(B=64, C=192, 28x28, w=14, 3x3 inter-block mix): the fused forward kernel (partition, M_c formed
on chip from the table, MFMA contraction, reverse, mix, saved pre-mix map), the fused backward
kernel (mix adjoint, dX = M^T G, row-pair MFMA table gradient, dWmix partials) and the small
fixed-order reduction kernel that finishes dT and dWmix.

Prints ONE JSON line on stdout; diagnostics go to stderr.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
      NAME: train_w14 (default), train_w14_hier (sub-window fold + dT_sub), train_w14_shift /
      train_stage1_shift (interleaved window grid at 28x28 / 56x56), train_w14_bf16 /
      train_w14_bf16_mix (bf16 maps), stage1_w14,
      bf16_w7 / bf16_w14 / bf16_w28, highres_w14, tiny_w7 (see receptive_field_spatial_amd/synth.py)
  python bench.py --workload stage1_w14 --cached   # forward on M cached in HBM
  python bench.py --copy-calibration        # plain device copy for HBM counter scaling
  python bench.py --fig3-sweep              # WBMM w=7/14/28 vs DW-Std k=5..13, one line each
  python bench.py --summarize-pmc DIR ...   # turn rocprofv3 --pmc output into profiles/ json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_MFMA_PEAK_TFLOPS = 157.3     # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 matrix
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E
# fp32 FMA on the vector ALUs without packed (two-wide) instructions, which these kernels do not
# use: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
METRIC = "WBMM fwd+bwd GFLOP/s & out-elems/s at w=14; % of MFMA/HBM roofline"
CSRC = os.path.join(ROOT, "receptive_field_spatial_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# kernel -> the source file that defines it. A kernel's hash covers that file and the device
# headers it includes (directly or through another header); wbmm_launch.hpp (host-side request
# structs and launcher declarations) and the other kernels' files do not change it.
KERNEL_FILES = {"k_fwd_ws": "wbmm_fast.hip", "k_bwd_ls": "wbmm_fast.hip", "k_fwd_cm": "wbmm_fastcm.hip",
                "k_fwd_bf16_w7": "wbmm_fastbf.hip",
                "k_fwd_bf16_w28": "wbmm_fastbf.hip", "k_fwd_bf16": "wbmm_fastbf.hip",
                "k_wbmm_fwd": "wbmm_fwd.hip", "k_wbmm_bwd": "wbmm_bwd.hip",
                "k_fwd_f32_w7": "wbmm_fast7.hip", "k_fwd_f32_w28": "wbmm_fast28.hip",
                "k_fwd_tab": "wbmm_fasttab.hip", "k_mix_direct": "wbmm_aux.hip",
                "k_roll_fwd": "wbmm_fastroll.hip", "k_roll_bwd": "wbmm_fastroll.hip"}
HOST_HEADERS = ("wbmm_launch.hpp",)


def _device_sources(name: str, seen=None):
    """`name` and the local headers it includes, transitively, minus the host-side ones."""
    seen = [] if seen is None else seen
    if name in seen or name in HOST_HEADERS:
        return seen
    seen.append(name)
    with open(os.path.join(CSRC, name), encoding="utf-8") as f:
        for inc in re.findall(r'^\s*#include\s+"([^"]+)"', f.read(), flags=re.M):
            _device_sources(inc, seen)
    return seen


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in sorted(_device_sources(KERNEL_FILES[kernel])):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _code_only(src: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so that editing a comment
    does not invalidate counters taken with the same code."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


# ----------------------------------------------------------------------------- accounting
def accounting(wl, cached=False):
    """Algorithmic flops and bytes (the method's minimum), per kernel and per step.

    flops: 2d per element of the window grid for the window contraction (a map whose sides are
    not multiples of w is computed on the zero-padded grid), 4d for its backward (dX + dT),
    18 per output element for the 3x3 mix and 36 for its backward (data + weight).
    bytes: every input read once, every output written once, plus the per-channel table (and
    the sub-window table when the fold is on; its gradient in the backward).
    """
    d = wl.w * wl.w
    E = wl.B * wl.C * wl.H * wl.W
    # the window grid the method computes: the map zero-padded up to whole windows. (The extra
    # border windows of an interleaved grid are counted as overhead, not work.)
    Hp = -(-wl.H // wl.w) * wl.w
    Wp = -(-wl.W // wl.w) * wl.w
    Eg = wl.B * wl.C * Hp * Wp
    esz = 2 if wl.dtype == "bf16" else 4
    L = (2 * wl.w - 1) ** 2
    tab = wl.C * L * esz
    if wl.s is not None:
        tab += wl.C * (2 * wl.s - 1) ** 2 * esz
    if cached:
        tab = wl.C * d * d * esz  # the cached (folded) matrices are read instead of the tables
    fwd_flops = Eg * 2 * d + E * (18 if wl.mix else 0)
    fwd_bytes = E * esz * (2 + (1 if wl.backward else 0)) + tab + (wl.C * 36 if wl.mix else 0)
    acc = {"E": E, "E_grid": Eg, "d": d, "fwd_flops": fwd_flops, "fwd_bytes": fwd_bytes}
    if wl.backward:
        acc["bwd_flops"] = Eg * 4 * d + E * (36 if wl.mix else 0)
        # reads x, dy, z (mix), table; writes dx, dT, dWmix
        acc["bwd_bytes"] = E * esz * (3 + (1 if wl.mix else 0)) + tab + wl.C * L * 4 + \
            (wl.C * 72 if wl.mix else 0)
    acc["step_flops"] = fwd_flops + acc.get("bwd_flops", 0)
    return acc


def mix_in_main_kernel(wl, cached=False):
    """Whether the main forward and backward kernels apply the 3x3 mix (and its adjoint)
    themselves: the w = 14 kernels on whole 14/28/56 images of the plain grid. Elsewhere the mix
    runs as a pass of its own."""
    whole = wl.w == 14 and wl.H == wl.W and wl.H in (14, 28, 56)
    return wl.mix and whole and not wl.shift and not cached


# ----------------------------------------------------------------------------- CPU baseline
def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = 10.0, cached: bool = False):
    """Time the oracle (as it is) on the same step, repeated until ~budget_s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import wbmm_oracle as O
    from receptive_field_spatial_amd import synth

    inp = synth.draw_inputs(wl)
    x = inp["x"].astype(np.float64)
    T = inp["T"].astype(np.float64)
    Wm = inp.get("Wmix")
    Ts = inp["T_sub"].astype(np.float64) if wl.s is not None else None
    dy = inp["dY"].astype(np.float64) if wl.backward else None
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if cached:  # inference with the cached (folded) matrix
            M = O.build_matrix(T, wl.w)
            if Ts is not None:
                M = O.fold_hier(M, Ts, wl.w, wl.s)
            O.layer_forward(x, wl.w, M=M, Wmix=Wm)
        elif wl.shift:
            y, z = O.layer_forward_shifted(x, wl.w, wl.shift, wl.shift, T=T, Wmix=Wm)
            if wl.backward:
                O.layer_backward_shifted(x, dy, wl.w, wl.shift, wl.shift, T=T, Wmix=Wm, z=z)
        elif Ts is not None:
            y, z = O.layer_forward_hier(x, wl.w, wl.s, T, Ts, Wmix=Wm)
            if wl.backward:
                O.layer_backward_hier(x, dy, wl.w, wl.s, T, Ts, Wmix=Wm, z=z)
        else:
            y, z = O.layer_forward(x, wl.w, T=T, Wmix=Wm)
            if wl.backward:
                O.layer_backward(x, dy, wl.w, T=T, Wmix=Wm, z=z)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s and len(times) >= 3:
            break
    med = statistics.median(times)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    acc = accounting(wl, cached)
    what = "fwd+bwd" if wl.backward else "fwd"
    return {
        "value": round(acc["step_flops"] / med / 1e9, 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": host_cpu_model(),
        "sample": f"full {wl.name} step ({what}, all {wl.C} channels), {len(times)} runs, median "
                  f"{med:.3f} s; fp64 numpy/OpenBLAS on {len(os.sched_getaffinity(0))} host CPUs",
    }


# ----------------------------------------------------------------------------- traffic
def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if taken on this source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("kernel_name") not in KERNEL_FILES:
        return None
    if k.get("src_hash") != kernel_source_hash(k["kernel_name"]):
        return None  # the kernel changed since the counters were taken
    return k.get("hbm_bytes_per_launch")


def profiled_kernel_name(workload: str, kernel: str):
    """The kernel that the committed counter run of this workload saw under a bench label."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        k = json.load(f).get("kernels", {}).get(kernel)
    return None if k is None else k.get("kernel_name")


# ----------------------------------------------------------------------------- HIP events
class HipEvents:
    """Raw hipEvent_t handles (the library records them around its main kernel launch)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(self.ct.c_void_p(ev))


# ----------------------------------------------------------------------------- measured peaks
def measure_peaks(R, torch, hev):
    """Peaks measured in the same session, beside the datasheet ones: the matrix-core probe
    (wbmm_probe_mfma: 8 independent MFMA chains per wave, 4096 waves, no memory traffic) for fp32
    and bf16, and a 1 GiB device-to-device copy (read + write bytes / time) for HBM. Best of 3."""
    out = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    peaks = {}
    for name, dt, iters in (("fp32_mfma_tflops", torch.float32, 2000),
                            ("bf16_mfma_tflops", torch.bfloat16, 2048)):
        best = 0.0
        for _ in range(3):
            a, b = hev.create(), hev.create()
            R.wbmm_set_launch_events(a, b)
            flops = R.wbmm_probe_mfma(dt, 1024, iters, out=out)
            torch.cuda.synchronize()
            best = max(best, flops / (hev.elapsed_ms(a, b) / 1e3) / 1e12)
            hev.destroy(a)
            hev.destroy(b)
        peaks[name] = round(best, 1)
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * n * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9)
    peaks["hbm_copy_gbs"] = round(best, 1)
    del src, dst
    return peaks


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


# ----------------------------------------------------------------------------- GPU run
def run(args):
    import numpy as np
    import torch

    import receptive_field_spatial_amd as R
    from receptive_field_spatial_amd import synth

    R.load_library()
    wl = synth.WORKLOADS[args.workload]
    if args.cached and (wl.backward or wl.shift):
        raise SystemExit("--cached applies to the forward-only workloads on the plain grid")
    acc = accounting(wl, args.cached)
    dev = torch.device("cuda:0")
    inp = synth.draw_inputs(wl)
    bf16 = wl.dtype == "bf16"

    def to_dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    # Rotate among independent input/output sets so that each step reads a batch that is not
    # already sitting in the 256 MB last-level cache (as in training, where batches change).
    nsets = max(1, args.rotate)
    sets = []
    for _ in range(nsets):
        s = {"x": to_dev(inp["x"])}
        s["y"] = torch.empty_like(s["x"])
        if wl.backward:
            s["dy"] = to_dev(inp["dY"])
            if wl.mix:
                s["z"] = torch.empty_like(s["x"])
            s["dx"] = torch.empty_like(s["x"])
        sets.append(s)
    T = to_dev(inp["T"])
    Wm = torch.from_numpy(inp["Wmix"]).to(dev) if wl.mix else None  # the mix weights stay fp32
    M = None
    Tsub = to_dev(inp["T_sub"]) if wl.s is not None else None
    hier_train = wl.s is not None and wl.backward  # fold on chip, dT_sub in the backward
    hier_chip = wl.s is not None and not args.cached  # the forward folds T_sub on chip
    if args.cached:  # inference caching: M (folded: M') built once, then read every step
        M = R.wbmm_build_matrix(T, wl.w)
        if wl.s is not None:
            M = R.wbmm_fold_hier(M, Tsub, wl.w, wl.s)
    L = 2 * wl.w - 1
    dT = torch.empty((wl.C, L, L), dtype=torch.float32, device=dev)
    dW = torch.empty((wl.C, 3, 3), dtype=torch.float32, device=dev) if wl.mix else None
    dTs = (torch.empty((wl.C, 2 * wl.s - 1, 2 * wl.s - 1), dtype=torch.float32, device=dev)
           if hier_train else None)
    ws_b = None
    bf16_bwd = bf16 and wl.backward
    if wl.backward:
        if bf16_bwd:
            nb = R.wbmm_backward_bf16_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, has_mix=wl.mix)
        elif wl.shift:
            nb = R.wbmm_backward_shifted_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, wl.shift,
                                                         wl.shift, has_mix=wl.mix)
        elif hier_train:
            nb = R.wbmm_backward_hier_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, wl.s,
                                                      has_mix=wl.mix)
        else:
            nb = R.wbmm_backward_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, has_mix=wl.mix)
        ws_b = torch.zeros(nb, dtype=torch.uint8, device=dev)
    if wl.shift:
        nf = R.wbmm_forward_shifted_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, wl.shift,
                                                    wl.shift, has_mix=wl.mix,
                                                    has_z_save=wl.backward and wl.mix)
    elif hier_chip:
        nf = R.wbmm_forward_hier_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, wl.s,
                                                 has_mix=wl.mix, has_z_save=wl.backward and wl.mix)
    else:
        nf = R.wbmm_forward_workspace_bytes(wl.B, wl.C, wl.H, wl.W, wl.w, has_mix=wl.mix,
                                            has_z_save=wl.backward and wl.mix)
    ws_f = torch.empty(max(nf, 1), dtype=torch.uint8, device=dev) if nf else None
    stream = torch.cuda.current_stream()
    kw_tab = {"M": M} if M is not None else {"T": T}

    def fwd(s):
        if wl.shift:
            R.wbmm_forward_shifted(s["x"], wl.w, wl.shift, wl.shift, mix_w=Wm, y=s["y"],
                                   z_save=s.get("z"), workspace=ws_f, stream=stream, **kw_tab)
            return
        if hier_chip:
            R.wbmm_forward_hier(s["x"], wl.w, wl.s, T, Tsub, mix_w=Wm, y=s["y"], z_save=s.get("z"),
                                workspace=ws_f, stream=stream)
            return
        R.wbmm_forward(s["x"], wl.w, mix_w=Wm, y=s["y"], z_save=s.get("z"), workspace=ws_f,
                       stream=stream, **kw_tab)

    def bwd(s):
        if bf16_bwd:
            R.wbmm_backward_bf16(s["x"], s["dy"], wl.w, T, mix_w=Wm,
                                 z_saved=s["z"] if wl.mix else None, dx=s["dx"], dT=dT,
                                 dmix_w=dW if wl.mix else False, workspace=ws_b, stream=stream)
            return
        if wl.shift:
            R.wbmm_backward_shifted(s["x"], s["dy"], wl.w, wl.shift, wl.shift, mix_w=Wm,
                                    z_saved=s["z"] if wl.mix else None, dx=s["dx"], dT=dT,
                                    dmix_w=dW if wl.mix else False, workspace=ws_b,
                                    stream=stream, **kw_tab)
            return
        if hier_train:
            R.wbmm_backward_hier(s["x"], s["dy"], wl.w, wl.s, T, Tsub, mix_w=Wm,
                                 z_saved=s["z"] if wl.mix else None, dx=s["dx"], dT=dT,
                                 dT_sub=dTs, dmix_w=dW if wl.mix else False, workspace=ws_b,
                                 stream=stream)
            return
        R.wbmm_backward(s["x"], s["dy"], wl.w, mix_w=Wm, z_saved=s["z"] if wl.mix else None,
                        dx=s["dx"], dT=dT, dmix_w=dW if wl.mix else False, workspace=ws_b,
                        stream=stream, **kw_tab)

    for i in range(args.warmup):
        s = sets[i % nsets]
        fwd(s)
        if wl.backward:
            bwd(s)
    torch.cuda.synchronize()

    K = args.steps
    hev = HipEvents()
    # timed region: K steps exactly as a caller runs them (no instrumentation)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        s = sets[i % nsets]
        fwd(s)
        if wl.backward:
            bwd(s)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / K
    # the same K steps again with HIP events around the main kernels on their launch stream (the
    # library records the pair it was handed around its main kernel's dispatch; the bf16 backward's
    # several kernels are bracketed here). Each event adds a few microseconds of queue work, so this
    # pass gives kernel durations, not the step time.
    kev = [[hev.create() for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    i0.record(stream)
    for i in range(K):
        s = sets[i % nsets]
        R.wbmm_set_launch_events(kev[i][0], kev[i][1])
        fwd(s)
        if wl.backward:
            if bf16_bwd:  # several kernels (dX contraction, row-pair dT, reduction): time them all
                hev.record(kev[i][2], stream)
                bwd(s)
                hev.record(kev[i][3], stream)
            else:
                R.wbmm_set_launch_events(kev[i][2], kev[i][3])
                bwd(s)
    i1.record(stream)
    torch.cuda.synchronize()
    ms_step_instr = i0.elapsed_time(i1) / K
    # main-kernel durations: the library attaches the events to each main kernel's dispatch
    fwd_ms = [hev.elapsed_ms(e[0], e[1]) for e in kev]
    bwd_ms = [hev.elapsed_ms(e[2], e[3]) for e in kev] if wl.backward else []
    for e in kev:
        for h in e:
            hev.destroy(h)
    # warm: the same input set every step (resident in the 256 MB last-level cache when it fits)
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(K):
        fwd(sets[0])
        if wl.backward:
            bwd(sets[0])
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / K
    peaks = measure_peaks(R, torch, hev)
    log(f"[bench] {wl.name}: {K} steps in {total_ms:.3f} ms GPU ({wall*1e3:.1f} ms wall); "
        f"fwd kernel avg {statistics.mean(fwd_ms)*1e3:.1f} us"
        + (f", bwd kernel avg {statistics.mean(bwd_ms)*1e3:.1f} us" if bwd_ms else ""))

    # dominant kernel and its roofline
    fwd_avg = statistics.mean(fwd_ms) / 1e3
    # the mix's flops count for the main kernel only where it applies the mix itself (the bf16
    # backward's bracket holds all of its kernels, the mix pass included)
    mixf = acc["E"] * 18 if wl.mix else 0
    fused = mix_in_main_kernel(wl, args.cached)
    kernels = {"k_wbmm_fwd": (fwd_avg, acc["fwd_flops"] - (0 if fused else mixf), acc["fwd_bytes"])}
    if wl.backward:
        kernels["k_wbmm_bwd"] = (statistics.mean(bwd_ms) / 1e3,
                                 acc["bwd_flops"] - (0 if fused or bf16_bwd else 2 * mixf),
                                 acc["bwd_bytes"])
    kname = max(kernels, key=lambda k: kernels[k][0])
    ksec, kflops, kbytes = kernels[kname]
    mfma_bound = not (bf16 and wl.w <= 14)
    if mfma_bound:
        peak = BF16_MFMA_PEAK_TFLOPS if bf16 else FP32_MFMA_PEAK_TFLOPS
        achieved = kflops / ksec / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = kbytes / ksec / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    meas = (peaks["hbm_copy_gbs"] if roof["bound"] == "hbm" else
            peaks["bf16_mfma_tflops"] if bf16 else peaks["fp32_mfma_tflops"])
    roof["peak_measured"] = meas
    roof["frac_of_measured"] = round(roof["achieved"] / meas, 4)
    roof["traffic"] = load_traffic(wl.name + ("_cached" if args.cached else ""), kname)
    roof["kernel"] = kname
    roof["kernel_profiled_as"] = profiled_kernel_name(wl.name + ("_cached" if args.cached else ""), kname)
    roof["kernel_us"] = round(ksec * 1e6, 2)
    roof["algorithmic_per_launch"] = kflops if mfma_bound else kbytes

    value = acc["step_flops"] / (ms_step / 1e3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W, "w": wl.w,
                   "mix": wl.mix, "fold_s": wl.s, "grid_offset": wl.shift,
                   "pass": "fwd+bwd" if wl.backward else "fwd",
                   "matrix": ("cached M" if M is not None else
                              "formed and folded on chip from T, T_sub" if hier_chip else
                              "formed on chip from T"),
                   "rotating_batches": nsets},
        "out_elems_per_s": round(acc["E"] / (ms_step / 1e3), 1),
        "grid_elems_per_s": round(acc["E_grid"] / (ms_step / 1e3), 1),
        "roofline": roof,
    }
    if wl.backward:
        line["kernels_us"] = {k: round(v[0] * 1e6, 2) for k, v in kernels.items()}
    kl = bwd_ms if kname == "k_wbmm_bwd" else fwd_ms
    roof["kernel_us_median_p10_p90"] = [round(statistics.median(kl) * 1e3, 2),
                                        round(_pct(kl, 0.1) * 1e3, 2), round(_pct(kl, 0.9) * 1e3, 2)]
    line["ms_per_step_warm"] = round(warm_ms, 4)
    line["ms_per_step_instrumented"] = round(ms_step_instr, 4)
    line["peaks_measured"] = peaks
    if args.cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget, args.cached)
    return line


# ----------------------------------------------------------------------------- profiling helpers
def copy_calibration(mib: int = 512):
    """A plain device-to-device copy of known size (read mib MiB, write mib MiB)."""
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[copy] {mib} MiB copied 3 times")


def _pmc_rows(d):
    """Counter rows of a rocprofv3 --pmc output directory (CSV or rocpd SQLite database)."""
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    for p in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        import sqlite3
        con = sqlite3.connect(p)
        try:
            for disp, kname, cname, val in con.execute(
                    "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
                rows.append({"Dispatch_Id": disp, "Kernel_Name": kname, "Counter_Name": cname,
                             "Counter_Value": val})
        finally:
            con.close()
    return rows


# bench label -> names of the kernels that can be that call's main kernel (fast or general path)
MAIN_KERNELS = {"k_wbmm_fwd": ("k_fwd_ws", "k_fwd_cm", "k_fwd_bf16_w7", "k_fwd_bf16_w28", "k_fwd_bf16",
                               "k_fwd_f32_w7", "k_fwd_f32_w28", "k_fwd_tab", "k_roll_fwd",
                               "k_wbmm_fwd"),
                "k_wbmm_bwd": ("k_bwd_ls", "k_roll_bwd", "k_wbmm_bwd")}


def _per_dispatch(rows, counter, names, with_name=False):
    """Median over dispatches of a counter summed over its rows, for the first of `names` that
    some dispatch's kernel name contains."""
    for n in names:
        vals = {}
        for r in rows:
            if r.get("Counter_Name") != counter or n not in r.get("Kernel_Name", ""):
                continue
            key = r.get("Dispatch_Id")
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        if vals:
            med = statistics.median(vals.values())
            return (med, n) if with_name else med
    return (None, None) if with_name else None


def summarize_pmc(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib=512):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> bytes, scaled by the copy kernel's reading."""
    true_kib = copy_mib * 1024.0
    cf = _per_dispatch(_pmc_rows(copy_fetch_dir), "FETCH_SIZE", ("copy",))
    cw = _per_dispatch(_pmc_rows(copy_write_dir), "WRITE_SIZE", ("copy",))
    f_fac = cf / true_kib
    w_fac = cw / true_kib
    rec = {"workload": workload,
           "copy_kernel": {"bytes_each_way": copy_mib * 2**20, "fetch_kib": cf, "write_kib": cw,
                           "fetch_factor": f_fac, "write_factor": w_fac},
           "kernels": {}}
    frows, wrows = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    for k, names in MAIN_KERNELS.items():
        fk, kname = _per_dispatch(frows, "FETCH_SIZE", names, with_name=True)
        wk = _per_dispatch(wrows, "WRITE_SIZE", (kname,)) if kname else None
        if fk is None or wk is None:
            continue
        rb = fk / f_fac * 1024.0
        wb = wk / w_fac * 1024.0
        rec["kernels"][k] = {"kernel_name": kname, "src_hash": kernel_source_hash(kname),
                             "fetch_kib_raw": fk, "write_kib_raw": wk, "read_bytes": rb,
                             "write_bytes": wb, "hbm_bytes_per_launch": rb + wb}
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    log(f"[pmc] wrote {out}")


# ----------------------------------------------------------------------------- DW-Std comparison
FIG3 = {"B": 128, "C": 256, "H": 56, "W": 56}


def fig3_sweep(args):
    """The pages' operator comparison on this GPU: one layer call at batch 128, 256 channels,
    56x56, fp32, for WBMM (w = 7, 14, 28; table input, no mix) and the k x k depthwise convolution
    (k = 5 .. 13). Each line: main-kernel time from HIP events on its dispatch (inputs rotate over
    4 batches), output elements/s (the same output for every operator), algorithmic GFLOP/s and
    the roofline of the binding resource."""
    import numpy as np
    import torch

    import receptive_field_spatial_amd as R
    from receptive_field_spatial_amd import synth

    R.load_library()
    B, C, H, W = FIG3["B"], FIG3["C"], FIG3["H"], FIG3["W"]
    E = B * C * H * W
    nsets = max(1, args.rotate)
    xs = [torch.from_numpy(synth.normal_f32((B, C, H, W), 1.0, seed=i)).cuda() for i in range(nsets)]
    ys = [torch.empty_like(xs[0]) for _ in range(nsets)]
    hev = HipEvents()
    stream = torch.cuda.current_stream()

    def timed(call):
        for i in range(args.warmup):
            call(i % nsets)
        torch.cuda.synchronize()
        evs = [(hev.create(), hev.create()) for _ in range(args.steps)]
        for i in range(args.steps):
            R.wbmm_set_launch_events(evs[i][0], evs[i][1])
            call(i % nsets)
        torch.cuda.synchronize()
        ms = [hev.elapsed_ms(a, b) for a, b in evs]
        for a, b in evs:
            hev.destroy(a)
            hev.destroy(b)
        return statistics.mean(ms) / 1e3

    lines = []
    for w in (7, 14, 28):
        T = torch.from_numpy(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=50 + w)).cuda()
        sec = timed(lambda i: R.wbmm_forward(xs[i], w, T=T, y=ys[i], stream=stream))
        Hp, Wp = -(-H // w) * w, -(-W // w) * w
        flops = B * C * Hp * Wp * 2 * w * w
        nbytes = E * 8 + C * (2 * w - 1) ** 2 * 4
        t_mfma = flops / (FP32_MFMA_PEAK_TFLOPS * 1e12)
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        roof = ({"bound": "mfma", "peak_tflops": FP32_MFMA_PEAK_TFLOPS,
                 "frac": round(t_mfma / sec, 4)} if t_mfma >= t_hbm else
                {"bound": "hbm", "peak_gbs": HBM_PEAK_GBS, "frac": round(t_hbm / sec, 4)})
        lines.append({"op": "wbmm", "w": w, "receptive_field": w * w, "us": round(sec * 1e6, 2),
                      "out_elems_per_s": round(E / sec, 1), "gflops": round(flops / sec / 1e9, 1),
                      "roofline": roof})
    # context beyond the pages' fp32 comparison: the same layers with bf16 maps and tables
    xb = [x.to(torch.bfloat16) for x in xs]
    yb = [torch.empty_like(x) for x in xb]
    for w in (7, 14, 28):
        T = torch.from_numpy(synth.normal_f32((C, 2 * w - 1, 2 * w - 1), 0.02, seed=50 + w)).cuda()
        Tb = T.to(torch.bfloat16)
        sec = timed(lambda i: R.wbmm_forward(xb[i], w, T=Tb, y=yb[i], stream=stream))
        flops = B * C * H * W * 2 * w * w
        nbytes = E * 4 + C * (2 * w - 1) ** 2 * 2
        t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        roof = ({"bound": "mfma", "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": round(t_mfma / sec, 4)} if t_mfma >= t_hbm else
                {"bound": "hbm", "peak_gbs": HBM_PEAK_GBS, "frac": round(t_hbm / sec, 4)})
        lines.append({"op": "wbmm_bf16", "w": w, "receptive_field": w * w,
                      "us": round(sec * 1e6, 2), "out_elems_per_s": round(E / sec, 1),
                      "gflops": round(flops / sec / 1e9, 1), "roofline": roof})
    del xb, yb
    for k in (5, 7, 9, 11, 13):
        Wd = torch.from_numpy(synth.normal_f32((C, k, k), 0.05, seed=60 + k)).cuda()
        sec = timed(lambda i: R.wbmm_dwconv_forward(xs[i], Wd, y=ys[i], stream=stream))
        flops = E * 2 * k * k
        nbytes = E * 8 + C * k * k * 4
        t_alu = flops / (FP32_VALU_PEAK_TFLOPS * 1e12)
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        roof = ({"bound": "alu", "peak_tflops": round(FP32_VALU_PEAK_TFLOPS, 1),
                 "frac": round(t_alu / sec, 4)} if t_alu >= t_hbm else
                {"bound": "hbm", "peak_gbs": HBM_PEAK_GBS, "frac": round(t_hbm / sec, 4)})
        lines.append({"op": "dw_std", "k": k, "receptive_field": k * k, "us": round(sec * 1e6, 2),
                      "out_elems_per_s": round(E / sec, 1), "gflops": round(flops / sec / 1e9, 1),
                      "roofline": roof})
    base = next(l for l in lines if l["op"] == "dw_std" and l["k"] == 5)["us"]
    for l in lines:
        l["speed_vs_dw5"] = round(base / l["us"], 3)
        l["config"] = dict(FIG3, dtype="bf16" if l["op"] == "wbmm_bf16" else "f32",
                           data="synthetic", rotating_batches=nsets)
        print(json.dumps(l), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="train_w14")
    ap.add_argument("--cached", action="store_true",
                    help="forward-only workloads: read M built once by wbmm_build_matrix "
                         "(inference caching) instead of forming it on chip from T")
    ap.add_argument("--rotate", type=int, default=4, help="independent batches cycled per step")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle CPU work")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--fig3-sweep", action="store_true",
                    help="WBMM vs DW-Std at batch 128, 256 channels, 56x56, fp32")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)
    if args.summarize_pmc:
        summarize_pmc(args.workload + ("_cached" if args.cached else ""), *args.summarize_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.fig3_sweep:
        fig3_sweep(args)
        return
    line = run(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
