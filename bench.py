#!/usr/bin/env python3
"""Benchmark of the PSA attention hot path on one MI355X.

One step = one pass of the whole path over one batch: psa_attn_fwd (O, LSE)
then psa_attn_bwd (D/LSE preprocess, dK/dV, dQ) on resident synthetic
inputs.  Prints ONE JSON line.

  value         backward TFLOP/s on the headline workload, algorithmic flops
                BH * 2N^2 (3dk + 2dv) over the backward's event-timed duration
  ms_per_step   wall time per fwd+bwd step (synchronised on both sides)
  roofline      the dominant kernel: algorithmic flops per launch / average
                launch duration from hipEvents recorded by the library around
                each launch on its stream, against the bf16 dense MFMA peak
  cpu_baseline  the float64 oracle timed on the host cores on a bounded
                sample of the same workload
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PSA attn bwd TFLOP/s + µs/call (B=16,N=400 & N=6400), % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # MI355X dense MFMA
# dense MFMA flops per clock per CU: 2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096
FLOP_PER_CLK_CU = {"bf16": 4096, "f16": 4096, "f32": 256}
PEAK_HBM_GBS = 8000.0
BATCHES = 5  # per-call times are the median over this many batches of K calls
HEADLINE = "highres_n6400_bf16"
ALSO = ("tiny_n64_f32", "nano_n400_f32", "batched_n400_bf16", "midres_n1600_bf16")  # the other four workloads


def flops(wl) -> dict:
    """Algorithmic flops per call for the whole batch (per (b,h) slice x BH)."""
    n2 = 2.0 * wl.N * wl.N * wl.BH
    return {
        "fwd": n2 * (wl.dk + wl.dv),                 # S = QK^T, O = PV
        "bwd": n2 * (3 * wl.dk + 2 * wl.dv),         # S recompute, dP, dV, dK, dQ
    }


def hbm_bytes(wl, e: int) -> dict:
    """Algorithmic HBM bytes per call (compulsory reads/writes, whole batch)."""
    N, BH, dk, dv = wl.N, wl.BH, wl.dk, wl.dv
    return {
        "fwd": BH * (e * N * (2 * dk + 2 * dv) + 4 * N),
        "bwd": BH * (e * N * (2 * (2 * dk + dv) + 2 * dv) + 4 * N),
        "bwd_pre": BH * (2 * e * N * dv + 4 * N + 8 * N),
    }


# every kernel source of the traced run (the traffic summary lists the
# convolution kernels too); build.py: the compile flags
KERNEL_SOURCES = ("psa_kernels.h", "psa_common.h", "psa_attn.hip", "psa_conv_kernels.h", "psa_conv_wide.h",
                  "psa_conv_wide.hip", "../build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_fingerprint() -> str:
    """Hash of the HIP sources and of the build script (its compile flags):
    counter-based traffic is reported only while it was measured on exactly
    these kernels."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vision_transformer_attention_psa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """Measured HBM bytes per launch {kernel: bytes} for `workload`, or None
    when absent or taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("fingerprint") != kernel_fingerprint():
        return None
    return rec.get("workloads", {}).get(workload)


def copy_calibration(torch, mib: int) -> None:
    """One elementwise pass dst = src * 1 over `mib` MiB of float32 (a kernel of
    known HBM traffic: mib MiB read, mib MiB written, far larger than the
    caches) used to scale the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def device_inputs(torch, x):
    import numpy as np
    from vision_transformer_attention_psa_amd import inputs
    if x.wl.dtype == inputs.BF16:
        q = torch.from_numpy(x.qkv_bits.view(np.int16)).view(torch.bfloat16).cuda()
        g = torch.from_numpy(x.dO_bits.view(np.int16)).view(torch.bfloat16).cuda()
    elif x.wl.dtype == inputs.F16:
        q = torch.from_numpy(x.qkv_bits.view(np.float16)).cuda()
        g = torch.from_numpy(x.dO_bits.view(np.float16)).cuda()
    else:
        q, g = torch.from_numpy(x.qkv).cuda(), torch.from_numpy(x.dO).cuda()
    return q, g


def device_peak(dtype: str) -> dict | None:
    """The dense MFMA peak recomputed from the device's own CU count and peak
    clock (hipDeviceGetAttribute), next to the published figure."""
    # the HIP runtime already in the process (torch's): loading another copy
    # would start a second runtime on the same device
    with open("/proc/self/maps") as f:
        paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln}
    if not paths:
        return None
    try:
        hip = ctypes.CDLL(sorted(paths)[0])
        val = ctypes.c_int()
        dev = ctypes.c_int()
        if hip.hipGetDevice(ctypes.byref(dev)) != 0:
            return None
        out = {}
        for name, attr in (("cus", 63), ("clock_khz", 5)):  # MultiprocessorCount, ClockRate
            if hip.hipDeviceGetAttribute(ctypes.byref(val), attr, dev) != 0:
                return None
            out[name] = val.value
    except OSError:
        return None
    out["tflops"] = out["cus"] * out["clock_khz"] * 1e3 * FLOP_PER_CLK_CU[dtype] / 1e12
    out["published_tflops"] = PEAK_TFLOPS[dtype]
    return out


def time_workload(torch, wl, steps: int, warmup: int) -> dict:
    """W untimed warm-up steps, then exactly K timed fwd+bwd steps (no library
    instrumentation), then BATCHES batches of K fwd-only and K bwd-only calls
    back to back (per-call time: the median over the batches), then K
    instrumented steps for per-kernel device times."""
    from vision_transformer_attention_psa_amd import binding, inputs
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(torch, x)
    o = torch.empty((wl.B, wl.heads, wl.dv, wl.N), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((wl.B, wl.heads, wl.N), dtype=torch.float32, device="cuda")
    d = torch.empty_like(qkv)

    def fwd():
        binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))

    def bwd():
        binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)

    binding.psa_attn_timing_enable(False)
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fwd_b, bwd_b = [], []
    for _ in range(BATCHES):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for _ in range(steps):
            fwd()
        ev[1].record()
        for _ in range(steps):
            bwd()
        ev[2].record()
        torch.cuda.synchronize()
        fwd_b.append(ev[0].elapsed_time(ev[1]) / steps)
        bwd_b.append(ev[1].elapsed_time(ev[2]) / steps)
    fwd_ms = statistics.median(fwd_b)
    bwd_ms = statistics.median(bwd_b)
    binding.psa_attn_timing_reset()
    binding.psa_attn_timing_enable(True)
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    binding.psa_attn_timing_enable(False)
    kern = binding.psa_attn_timing_read()
    assert torch.isfinite(d.float()).all().item(), "non-finite gradient"
    fl = flops(wl)
    dt = wl.dtype
    peak = PEAK_TFLOPS[dt]
    by = hbm_bytes(wl, 4 if dt == inputs.F32 else 2)
    avg = {k: (ms / n if n else float("nan")) for k, (ms, n) in kern.items()}
    return {
        "inputs": x,
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "fwd_us": fwd_ms * 1e3,
        "bwd_us": bwd_ms * 1e3,
        "batch_us": {"fwd": [v * 1e3 for v in fwd_b], "bwd": [v * 1e3 for v in bwd_b]},
        "fwd_GBps": by["fwd"] / (fwd_ms * 1e-3) / 1e9,
        "bwd_GBps": by["bwd"] / (bwd_ms * 1e-3) / 1e9,
        "fwd_frac_hbm_peak": by["fwd"] / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "bwd_frac_hbm_peak": by["bwd"] / (bwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "fwd_tflops": fl["fwd"] / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": fl["bwd"] / (bwd_ms * 1e-3) / 1e12,
        "fwd_bwd_tflops": (fl["fwd"] + fl["bwd"]) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12,
        "bwd_pct_mfma_peak": 100.0 * fl["bwd"] / (bwd_ms * 1e-3) / 1e12 / peak,
        "fwd_bwd_pct_mfma_peak": 100.0 * (fl["fwd"] + fl["bwd"]) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12 / peak,
        "kernel_avg_us": {k: v * 1e3 for k, v in avg.items()},
        "peak_tflops": peak,
        "dtype": dt,
    }


def time_workload_graph(torch, wl, steps: int, warmup: int) -> dict:
    """The fwd and the bwd call each captured once into a HIP graph and
    replayed K times: per-call time without Python/ctypes launch overhead.
    For kernels shorter than a graph launch the host stays the limit."""
    from vision_transformer_attention_psa_amd import binding, inputs
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(torch, x)
    o = torch.empty((wl.B, wl.heads, wl.dv, wl.N), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((wl.B, wl.heads, wl.N), dtype=torch.float32, device="cuda")
    d = torch.empty_like(qkv)
    binding.psa_attn_timing_enable(False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the scratch cache for the capture stream
        binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
        binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gf, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gf, stream=s):
        binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
    with torch.cuda.graph(gb, stream=s):
        binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    # the same calls K times in one graph: one graph launch per K calls
    gfk, gbk = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gfk, stream=s):
        for _ in range(steps):
            binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
    with torch.cuda.graph(gbk, stream=s):
        for _ in range(steps):
            binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    for _ in range(warmup):
        gf.replay()
        gb.replay()
    gfk.replay()
    gbk.replay()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    e[0].record()
    for _ in range(steps):
        gf.replay()
    e[1].record()
    for _ in range(steps):
        gb.replay()
    e[2].record()
    gfk.replay()
    e[3].record()
    gbk.replay()
    e[4].record()
    torch.cuda.synchronize()
    fl = flops(wl)
    fwd_us = e[0].elapsed_time(e[1]) * 1e3 / steps
    bwd_us = e[1].elapsed_time(e[2]) * 1e3 / steps
    return {"fwd_us": fwd_us, "bwd_us": bwd_us, "bwd_tflops": fl["bwd"] / (bwd_us * 1e-6) / 1e12,
            "calls_per_graph": steps, "fwd_us_in_one_graph": e[2].elapsed_time(e[3]) * 1e3 / steps,
            "bwd_us_in_one_graph": e[3].elapsed_time(e[4]) * 1e3 / steps}


COLD_FLUSH_MIB = 512  # twice the 256 MB last-level cache (Infinity Cache)


def time_workload_cold(torch, wl, steps: int) -> dict:
    """Each fwd and bwd call timed alone with hipEvents right after a 512 MiB
    buffer was overwritten, so that none of its inputs (nor O, LSE) is left
    in L2 or the last-level cache ("cold"), and the same loop without the
    overwrite ("warm_same_events"): each call carries one event pair, which
    at a few microseconds per call adds a visible share to both."""
    from vision_transformer_attention_psa_amd import binding, inputs
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(torch, x)
    o = torch.empty((wl.B, wl.heads, wl.dv, wl.N), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((wl.B, wl.heads, wl.N), dtype=torch.float32, device="cuda")
    d = torch.empty_like(qkv)
    flush = torch.empty(COLD_FLUSH_MIB << 20, dtype=torch.uint8, device="cuda")
    binding.psa_attn_timing_enable(False)
    binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
    binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    res = {}
    for mode in ("cold", "warm_same_events"):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in ev:
            if mode == "cold":
                flush.fill_(1)
            e[0].record()
            binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
            e[1].record()
            if mode == "cold":
                flush.fill_(2)
            e[2].record()
            binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
            e[3].record()
        torch.cuda.synchronize()
        fwd_us = sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3 / steps
        bwd_us = sum(e[2].elapsed_time(e[3]) for e in ev) * 1e3 / steps
        res[mode] = {"fwd_us": fwd_us, "bwd_us": bwd_us,
                     "bwd_tflops": flops(wl)["bwd"] / (bwd_us * 1e-6) / 1e12}
    res["flush_mib"] = COLD_FLUSH_MIB
    return res


def time_conv(torch, wl, steps: int, warmup: int) -> dict:
    """Backward of the block's qkv projection (a 1x1 convolution) at the
    workload's shape: x [B, heads*dv, N], w [heads*(2dk+dv), heads*dv], dy the
    packed gradient.  Two GEMMs of 2*B*N*cin*cout flops each."""
    import numpy as np
    from vision_transformer_attention_psa_amd import binding, inputs
    cin, cout = wl.heads * wl.dv, wl.heads * wl.channels
    ci = inputs.make_conv_inputs(wl.B, cin, cout, wl.N, wl.dtype, seed=wl.seed)

    def dev(a, k):
        if ci.bits is None:
            return torch.from_numpy(a).cuda()
        if wl.dtype == inputs.BF16:
            return torch.from_numpy(ci.bits[k].view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(ci.bits[k].view(np.float16)).cuda()

    x, w, dy = dev(ci.x, 0), dev(ci.w, 1), dev(ci.dy, 2)
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    binding.psa_attn_timing_enable(False)
    for _ in range(warmup):
        binding.conv_bwd(x, w, dy, out=(dx, dw))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        binding.conv_bwd(x, w, dy, out=(dx, dw))
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    binding.psa_attn_timing_reset()
    binding.psa_attn_timing_enable(True)
    for _ in range(steps):
        binding.conv_bwd(x, w, dy, out=(dx, dw))
    torch.cuda.synchronize()
    binding.psa_attn_timing_enable(False)
    kern = binding.psa_attn_timing_read()
    fl = 2 * 2.0 * wl.B * wl.N * cin * cout
    peak = PEAK_TFLOPS[wl.dtype]
    k_us = {k: kern[k][0] / kern[k][1] * 1e3 for k in ("conv_dx", "conv_dw") if kern[k][1]}
    return {"shape": {"B": wl.B, "cin": cin, "cout": cout, "N": wl.N}, "us_per_call": us,
            "tflops": fl / (us * 1e-6) / 1e12, "pct_mfma_peak": 100.0 * fl / (us * 1e-6) / 1e12 / peak,
            "kernel_avg_us": k_us,
            "kernel_tflops": {k: fl / 2 / (v * 1e-6) / 1e12 for k, v in k_us.items()}}


def time_cat(torch, wl, steps: int, warmup: int) -> dict:
    """Channel-concatenation backward at the workload's feature map: dy is
    the gradient of a concatenation of two [B, heads*dv, H, W] inputs (bf16 /
    the workload's dtype); one input's half is copied out (HBM-bound: each
    element read once and written once).  Then the copy folded into the qkv
    convolution's backward, whose input is such a concatenation, against the
    unfolded sequence (convolution backward, then one copy per part)."""
    from vision_transformer_attention_psa_amd import binding, inputs
    c = wl.heads * wl.dv
    tdt = {inputs.F32: torch.float32, inputs.BF16: torch.bfloat16, inputs.F16: torch.float16}[wl.dtype]
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    dy = torch.randn((wl.B, 2 * c, wl.N), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    dx = torch.empty((wl.B, c, wl.N), device="cuda", dtype=tdt)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    copy = lambda: binding.channel_cat_bwd(dy, c, c, out=dx)
    us = timed(copy)
    binding.psa_attn_timing_reset()
    binding.psa_attn_timing_enable(True)
    for _ in range(steps):
        copy()
    torch.cuda.synchronize()
    binding.psa_attn_timing_enable(False)
    kern = binding.psa_attn_timing_read()["cat"]
    k_us = kern[0] / kern[1] * 1e3
    nbytes = 2 * dx.numel() * dx.element_size()
    # Back-to-back calls bound the kernel time from above; the per-launch
    # event pair adds about 2 us, a fifth of this short kernel, so the
    # bandwidth is reported from the back-to-back time.
    gbs = nbytes / (us * 1e-6) / 1e9
    # the fold: x = cat(x_0, x_1) of c/2 channels each feeds the qkv convolution
    cout = wl.heads * wl.channels
    x = torch.randn((wl.B, c, wl.N), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    w = (torch.randn((cout, c), generator=g, device="cuda", dtype=torch.float32) / c ** 0.5).to(tdt)
    cdy = torch.randn((wl.B, cout, wl.N), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    full, dw = torch.empty_like(x), torch.empty_like(w)
    parts = [torch.empty((wl.B, c // 2, wl.N), device="cuda", dtype=tdt) for _ in range(2)]

    def unfolded():
        binding.conv_bwd(x, w, cdy, out=(full, dw))
        for k, p in enumerate(parts):
            binding.channel_cat_bwd(full, c // 2, k * (c // 2), out=p)

    folded_us = timed(lambda: binding.conv_cat_bwd(x, w, cdy, [c // 2, c // 2], out=(parts, dw)))
    unfolded_us = timed(unfolded)
    return {"copy": {"shape": {"B": wl.B, "channels": 2 * c, "slice": [c, 2 * c], "N": wl.N},
                     "us_per_call": us, "kernel_avg_us_with_event_gap": k_us, "bytes": nbytes,
                     "GB_per_s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS},
            "conv_fold": {"parts": [c // 2, c // 2], "folded_us": folded_us, "unfolded_us": unfolded_us}}


def time_lohi(torch, wl, steps: int, warmup: int) -> dict | None:
    """The two-call pattern (one attention call per half of V, merge, merge
    backward, two accumulating backward calls) at the workload's shape, next
    to the single call over all of V that computes the same results."""
    from vision_transformer_attention_psa_amd import binding, inputs
    h = wl.dv // 2
    code = {inputs.F32: binding.PSA_F32, inputs.BF16: binding.PSA_BF16, inputs.F16: binding.PSA_F16}[wl.dtype]
    if not binding.psa_attn_supported(wl.dk, h, code):
        return None
    qkv, dO = device_inputs(torch, inputs.make_inputs(wl))
    o_lo, l_lo = binding.fwd_vslice(qkv, wl.dk, wl.dv, 0, h, wl.scale)
    o_hi, l_hi = binding.fwd_vslice(qkv, wl.dk, wl.dv, h, wl.dv - h, wl.scale)
    merged = binding.merge_fwd(o_lo, o_hi)
    g_lo, g_hi = binding.merge_bwd(dO)
    d = torch.empty_like(qkv)

    def fwd():
        binding.fwd_vslice(qkv, wl.dk, wl.dv, 0, h, wl.scale, out=(o_lo, l_lo))
        binding.fwd_vslice(qkv, wl.dk, wl.dv, h, wl.dv - h, wl.scale, out=(o_hi, l_hi))
        binding.merge_fwd(o_lo, o_hi, out=merged)

    def bwd():
        binding.merge_bwd(dO, out=(g_lo, g_hi))
        binding.bwd_vslice(qkv, o_lo, l_lo, g_lo, d, wl.dk, wl.dv, 0, h, wl.scale, accumulate=False)
        binding.bwd_vslice(qkv, o_hi, l_hi, g_hi, d, wl.dk, wl.dv, h, wl.dv - h, wl.scale, accumulate=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    return {"halves": [h, wl.dv - h], "fwd_us": timed(fwd), "bwd_us": timed(bwd)}


def time_torch_sdpa(torch, wl, x, steps: int, warmup: int) -> dict | None:
    """For context only: torch's fused attention (scaled_dot_product_attention
    restricted to one backend at a time, so that nothing falls back to the
    unfused math path) on the same inputs, converted to its token-major
    [B, heads, N, d] layout outside the timed region.  Needs dk == dv (torch
    has no fused kernel otherwise).  Backward = (forward + backward) -
    forward, both timed with hipEvents over `steps` calls."""
    from vision_transformer_attention_psa_amd import inputs
    if wl.dk != wl.dv or wl.dtype == inputs.F32:
        return None
    from torch.nn.attention import SDPBackend, sdpa_kernel
    qkv, dO = x
    tok = lambda t: t.transpose(-1, -2).contiguous()
    q, k, v = (tok(qkv[:, :, a:a + wl.dk]) for a in (0, wl.dk, 2 * wl.dk))
    go = tok(dO)
    res = {"layout": "token-major [B, heads, N, d]", "note": "platform library, for context; not this library"}
    for backend in (SDPBackend.EFFICIENT_ATTENTION, SDPBackend.FLASH_ATTENTION):
        try:
            with sdpa_kernel([backend]):
                qq, kk, vv = (t.detach().requires_grad_() for t in (q, k, v))
                fwd = lambda: torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=wl.scale)

                def both():
                    fwd().backward(go)
                us = {}
                for name, fn in (("fwd", fwd), ("fwd_bwd", both)):
                    for _ in range(warmup):
                        fn()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record()
                    for _ in range(steps):
                        fn()
                    e1.record()
                    torch.cuda.synchronize()
                    us[name] = e0.elapsed_time(e1) * 1e3 / steps
                res[backend.name.lower()] = {"fwd_us": us["fwd"], "bwd_us": us["fwd_bwd"] - us["fwd"]}
        except Exception as e:  # the backend may be unavailable on a given build
            res[backend.name.lower()] = {"unavailable": f"{type(e).__name__}: {str(e)[:160]}"}
    return res


def roofline(wl, r: dict, traffic: dict | None) -> dict:
    """Dominant kernel of the step (largest average duration)."""
    fl = flops(wl)
    us = r["kernel_avg_us"]
    per_launch = {"fwd": fl["fwd"], "bwd_main": fl["bwd"]}  # one backward launch computes dQ, dK and dV
    name = max(per_launch, key=lambda k: us[k])
    achieved = per_launch[name] / (us[name] * 1e-6) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": achieved, "peak": r["peak_tflops"],
            "unit": "TFLOP/s", "frac": achieved / r["peak_tflops"], "avg_us": us[name],
            "flops_per_launch": per_launch[name],
            "traffic": (traffic or {}).get(name),
            "traffic_unit": "bytes/launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)"}


def _oracle_threads() -> tuple[int, int]:
    """(threads the oracle's BLAS actually runs, host cores this process may
    use).  The BLAS pool is sized by the environment (OMP_NUM_THREADS); it
    cannot run more threads at once than the cores the process may use."""
    host = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas = 1
    return min(blas, host), host


def _time_oracle(wl, x, budget_s: float) -> dict:
    """The float64 oracle on whole (b,h) slices of the draw x (the very
    inputs the GPU was timed on), in slice order, until about budget_s
    seconds of work have run (at least one slice)."""
    from oracle import psa_oracle as orc
    fl = flops(wl.with_(B=1, heads=1))
    fwd_s = bwd_s = 0.0
    n = 0
    while n < wl.BH and (n == 0 or fwd_s + bwd_s < budget_s):
        b, h = divmod(n, wl.heads)
        q = x.qkv[b:b + 1, h:h + 1]
        g = x.dO[b:b + 1, h:h + 1]
        t0 = time.perf_counter()
        o, lse = orc.forward(q, wl.dk, wl.dv, wl.scale)
        t1 = time.perf_counter()
        orc.backward(q, o, lse, g, wl.dk, wl.dv, wl.scale)
        t2 = time.perf_counter()
        fwd_s += t1 - t0
        bwd_s += t2 - t1
        n += 1
    return {"slices": n, "of": wl.BH, "fwd_ms_per_slice": fwd_s / n * 1e3, "bwd_ms_per_slice": bwd_s / n * 1e3,
            "bwd_tflops": fl["bwd"] * n / bwd_s / 1e12,
            "fwd_us_per_call": fwd_s / n * wl.BH * 1e6, "bwd_us_per_call": bwd_s / n * wl.BH * 1e6}


def cpu_baseline(wl, x, budget_s: float, others: dict) -> dict:
    """The oracle as it stands, on the host, on the same seeded inputs the
    GPU timed: the headline workload for about budget_s seconds, and each
    other workload in `others` ({name: (workload, inputs)}) for a few
    seconds at most."""
    used, host = _oracle_threads()
    head = _time_oracle(wl, x, budget_s)
    per = {name: _time_oracle(w, xi, min(4.0, budget_s)) for name, (w, xi) in others.items()}
    return {"value": head["bwd_tflops"], "unit": "TFLOP/s", "cores": used, "host_cores": host,
            "kind": "oracle",
            "sample": f"{head['slices']} of {wl.BH} (b,h) slices of {wl.name} (N={wl.N}, dk={wl.dk}, "
                      f"dv={wl.dv}), the same seeded draw the GPU timed; float64 numpy, BLAS on "
                      f"{used} threads ({host} host cores available); bwd "
                      f"{head['bwd_ms_per_slice']:.0f} ms/slice, fwd {head['fwd_ms_per_slice']:.0f} ms/slice",
            "bwd_us_per_call_extrapolated": head["bwd_us_per_call"],
            "fwd_us_per_call_extrapolated": head["fwd_us_per_call"],
            "per_workload": per}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--also", default=",".join(ALSO), help="comma list of extra workloads ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--graph", type=int, default=1, help="also time HIP-graph replay of the step (1/0)")
    ap.add_argument("--sdpa", type=int, default=1,
                    help="also time torch's fused attention on the headline inputs, for context (1/0)")
    ap.add_argument("--cold", type=int, default=0,
                    help="also time each call after overwriting 512 MiB (cold caches; 1/0). Off by default "
                         "so that a profile of the default command holds warm calls only")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one plain MIB-MiB device copy first (reference kernel for counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); every (batch, head) slice is independent and the multi-GPU "
              "split is a host-side partition of B*heads, which is not benchmarked here.",
              file=sys.stderr)
        return 2

    import torch
    from vision_transformer_attention_psa_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    wl = inputs.WORKLOADS[args.workload]
    print(f"[bench] {wl.name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    r = time_workload(torch, wl, args.steps, args.warmup)
    print(f"[bench] {wl.name}: fwd {r['fwd_us']:.1f} us, bwd {r['bwd_us']:.1f} us, "
          f"bwd {r['bwd_tflops']:.1f} TFLOP/s, kernels {r['kernel_avg_us']}", file=sys.stderr, flush=True)
    also, drawn = {}, {}
    for name in [a for a in args.also.split(",") if a]:
        a = time_workload(torch, inputs.WORKLOADS[name], args.steps, args.warmup)
        drawn[name] = (inputs.WORKLOADS[name], a["inputs"])
        also[name] = {k: a[k] for k in ("fwd_us", "bwd_us", "bwd_tflops", "bwd_pct_mfma_peak",
                                        "fwd_bwd_tflops", "fwd_bwd_pct_mfma_peak", "fwd_GBps", "bwd_GBps",
                                        "fwd_frac_hbm_peak", "bwd_frac_hbm_peak", "kernel_avg_us", "batch_us")}
        print(f"[bench] {name}: fwd {a['fwd_us']:.1f} us, bwd {a['bwd_us']:.1f} us, "
              f"bwd {a['bwd_tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    graph = {}
    if args.graph:
        for name in [wl.name] + [a for a in args.also.split(",") if a]:
            graph[name] = time_workload_graph(torch, inputs.WORKLOADS[name], args.steps, args.warmup)
            print(f"[bench] graph replay {name}: fwd {graph[name]['fwd_us']:.1f} us, "
                  f"bwd {graph[name]['bwd_us']:.1f} us; {args.steps} calls in one graph: fwd "
                  f"{graph[name]['fwd_us_in_one_graph']:.1f} us, bwd {graph[name]['bwd_us_in_one_graph']:.1f} us "
                  "per call", file=sys.stderr, flush=True)
    cold = {}
    for name in ([wl.name] + [a for a in args.also.split(",") if a]) if args.cold else []:
        cold[name] = time_workload_cold(torch, inputs.WORKLOADS[name], args.steps)
        c, w = cold[name]["cold"], cold[name]["warm_same_events"]
        print(f"[bench] cold caches {name}: fwd {c['fwd_us']:.1f} us, bwd {c['bwd_us']:.1f} us "
              f"(warm, same events: {w['fwd_us']:.1f} / {w['bwd_us']:.1f} us)", file=sys.stderr, flush=True)
    conv = time_conv(torch, wl, args.steps, args.warmup)
    print(f"[bench] qkv 1x1-conv backward {conv['shape']}: {conv['us_per_call']:.1f} us, "
          f"{conv['tflops']:.1f} TFLOP/s, kernels {conv['kernel_avg_us']}", file=sys.stderr, flush=True)
    cat = time_cat(torch, wl, args.steps, args.warmup)
    print(f"[bench] channel-cat backward {cat['copy']['shape']}: {cat['copy']['us_per_call']:.1f} us, "
          f"{cat['copy']['GB_per_s']:.0f} GB/s; folded into the conv backward "
          f"{cat['conv_fold']['folded_us']:.1f} us vs {cat['conv_fold']['unfolded_us']:.1f} us unfolded",
          file=sys.stderr, flush=True)
    lohi = time_lohi(torch, wl, args.steps, args.warmup)
    if lohi:
        print(f"[bench] lo/hi two-call pattern (halves {lohi['halves']}): fwd {lohi['fwd_us']:.1f} us, "
              f"bwd {lohi['bwd_us']:.1f} us (one call: fwd {r['fwd_us']:.1f}, bwd {r['bwd_us']:.1f})",
              file=sys.stderr, flush=True)
    sdpa = None
    if args.sdpa:
        sdpa = time_torch_sdpa(torch, wl, device_inputs(torch, r["inputs"])[:2], args.steps, args.warmup)
        if sdpa:
            print("[bench] torch fused attention (context) " + ", ".join(
                f"{k}: fwd {v['fwd_us']:.1f} us, bwd {v['bwd_us']:.1f} us" if "fwd_us" in v else f"{k}: unavailable"
                for k, v in sdpa.items() if isinstance(v, dict)), file=sys.stderr, flush=True)
    traffic = load_traffic(wl.name)
    cpu = None
    if args.cpu_budget > 0:
        print(f"[bench] cpu baseline: oracle on {wl.name} slices (~{args.cpu_budget:.0f} s)",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, r["inputs"], args.cpu_budget, drawn)
    out = {
        "metric": METRIC,
        "value": r["bwd_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic (seeded i.i.d. normal, bf16-rounded)",
        "config": {"workload": wl.name, "B": wl.B, "heads": wl.heads, "N": wl.N, "dk": wl.dk,
                   "dv": wl.dv, "step": "psa_attn_fwd + psa_attn_bwd"},
        "bwd_us_per_call": r["bwd_us"],
        "bwd_pct_mfma_peak": r["bwd_pct_mfma_peak"],
        "fwd_us_per_call": r["fwd_us"],
        "fwd_bwd_tflops": r["fwd_bwd_tflops"],
        "fwd_bwd_pct_mfma_peak": r["fwd_bwd_pct_mfma_peak"],
        "fwd_GBps": r["fwd_GBps"],
        "bwd_GBps": r["bwd_GBps"],
        "fwd_frac_hbm_peak": r["fwd_frac_hbm_peak"],
        "bwd_frac_hbm_peak": r["bwd_frac_hbm_peak"],
        "batch_us": r["batch_us"],
        "device_peak": device_peak(r["dtype"]),
        "kernel_avg_us": r["kernel_avg_us"],
        "roofline": roofline(wl, r, traffic),
        "cpu_baseline": cpu,
        "also": also,
        "graph_replay": graph,
        "cold_caches": cold,
        "qkv_conv_bwd": conv,
        "channel_cat_bwd": cat,
        "lo_hi_two_call": lohi,
        "torch_sdpa_reference": sdpa,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
