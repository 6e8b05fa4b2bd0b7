#!/usr/bin/env python
"""Attention forward + backward throughput on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
fa_fwd (O and LSE, online softmax, causal tile skipping) followed by fa_bwd
(Delta, dK/dV and dQ kernels with on-chip recomputation).  The default
workload is the long-context causal training problem B=1, H=16, N=65536,
D=64, bf16, seeded i.i.d. N(0, 1) inputs already resident in HBM.

Prints ONE JSON line.  ``value`` is algorithmic TFLOP/s of the step:
forward 4*B*H*N^2*D and backward 10*B*H*N^2*D, both halved under the causal
mask, divided by the mean step time measured with HIP events on the launch
stream (``step_ms`` adds the median and minimum of the per-step times).  The
``roofline`` object covers the kernel that takes the most time; its average
duration comes from per-launch HIP events that the library records on the
same stream during a second run of as many steps (kept out of the headline
steps).  ``sclk`` is the shader clock the driver reports while further steps
run back to back after both timed regions (the chip holds a clock below its
2.4 GHz peak at its power limit), and the ``*_at_measured_clock`` fields
scale the peak to it.  ``secondary`` times other workloads launch by launch (c2, c3, the
D = 128 forwards at N = 4096, 8192 and 16384, a D = 128 training step).
``cpu_baseline`` times the float64 oracle on a bounded sample (the leading
R x R causal block of head 0) on the host cores, with an extrapolation of
the whole workload's oracle time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(w):
    f = 4.0 * w.B * w.H * w.N * w.N * w.D
    b = 10.0 * w.B * w.H * w.N * w.N * w.D if w.backward else 0.0
    if w.causal:
        f, b = f / 2, b / 2
    return f, b


def kernel_algorithmic(w):
    """Algorithmic work of one launch of each kernel.  Contractions count
    2*N^2*D per head (halved when causal); the dQ kernel is credited with
    dQ = dS K only (its recomputation of S and dP is not algorithmic work);
    Delta is credited with its bytes (read O, dO; write Delta)."""
    unit = 2.0 * w.B * w.H * w.N * w.N * w.D * (0.5 if w.causal else 1.0)
    el = 2 if w.dtype in ("bf16", "f16") else 4
    return {
        "fwd": ("mfma", 2 * unit),           # S = Q K^T, O = P V
        "bwd_delta": ("hbm", 2.0 * w.B * w.H * w.N * w.D * el + 4.0 * w.B * w.H * w.N),
        "bwd_dkdv": ("mfma", 4 * unit),      # S, dP, dV, dK
        "bwd_dq": ("mfma", 1 * unit),        # dQ
        "bwd_dkdv_dq": ("mfma", 5 * unit),   # both in one launch (small D = 64 grids)
        # merge of two partials: read O, O_part, LSE, LSE_part; write O, LSE
        "merge": ("hbm", 3.0 * w.B * w.H * w.N * (w.D * el + 4)),
    }


KERNEL_SOURCES = {
    "fwd": ["fa_fwd.hip", "fa_device.h"],
    "bwd_delta": ["fa_bwd.hip", "fa_device.h"],
    "bwd_dkdv": ["fa_bwd.hip", "fa_bwd_dkdv.h", "fa_bwd_d128.hip", "fa_device.h"],
    "bwd_dq": ["fa_bwd.hip", "fa_device.h"],
    "bwd_dkdv_dq": ["fa_bwd.hip", "fa_bwd_dkdv.h", "fa_device.h"],
    "merge": ["fa_merge.hip", "fa_device.h"],
}


def source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_io_aware_58_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when there is none or the kernel's source
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}.md")
    if not os.path.exists(path):
        return None
    want = source_sha(kernel)
    for line in open(path, encoding="utf-8"):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == kernel and cells[6] == want:
            return float(cells[4]) + float(cells[5])
    return None


def upload(raw, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(raw)).cuda()


def run_gpu(w, steps, warmup, clock=None, clock_window_s=3.5):
    """Headline: `warmup` untimed steps, then `steps` steps between a
    synchronisation and an event on each side, one event between consecutive
    steps (per-step durations for the median and minimum); per-kernel event
    timing is off here.  Then the same number of steps again with the
    library's per-kernel events on, for the per-kernel averages.  Then, with
    a ClockSampler, steps back to back for `clock_window_s` seconds while it
    reads the shader clock.  Returns (ms per step, per-step times, per-kernel
    dict, ms per step of the second pass, clock summary or None)."""
    import torch
    from exact_io_aware_58_amd import fa, inputs

    log(f"[bench] inputs {w.name} {w.shape} {w.dtype} causal={w.causal}")
    devs = {n: upload(raw, w.dtype) for n, (_, raw) in inputs.make_inputs(w).items()}
    q, k, v = devs["q"], devs["k"], devs["v"]
    code = {"f32": fa.FA_F32, "bf16": fa.FA_BF16, "f16": fa.FA_F16}[w.dtype]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    if w.backward:
        do = devs["do"]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        wsb = fa.fa_bwd_workspace_bytes(code, w.B, w.H, w.N, w.D, w.causal)
        ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    args_f = (code, w.B, w.H, w.N, w.D, w.scale, w.causal, q.data_ptr(), k.data_ptr(),
              v.data_ptr(), o.data_ptr(), lse.data_ptr(), sh)
    if w.backward:
        args_b = (code, w.B, w.H, w.N, w.D, w.scale, w.causal, q.data_ptr(), k.data_ptr(),
                  v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                  dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), wsb, sh)

    def step():
        rc = fa.fa_fwd(*args_f)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_fwd")
        if w.backward:
            rc = fa.fa_bwd(*args_b)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, "fa_bwd")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup} done; timing {steps} steps")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    log(f"[bench] {steps} steps in {total_ms:.3f} ms")

    kreps = max(steps, 3)
    fa.fa_timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(kreps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    timed_ms = e0.elapsed_time(e1) / kreps
    clk = None
    if clock is not None and clock_window_s > 0:
        # the clock the chip holds under this load: more steps back to back
        # (outside both timed regions) while the sampler reads the driver
        clock.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < clock_window_s:
            for _ in range(4):
                step()
            torch.cuda.synchronize()
        clock.stop()
        clk = clock.summary(time.perf_counter() - t0)
    kernels = {}
    for kid in range(fa.FA_KERNEL_COUNT):
        n, ms, dropped = fa.fa_timing_read(kid)
        if n:
            kernels[fa.fa_kernel_name(kid)] = {"launches": n, "avg_ms": ms / n}
    fa.fa_timing_enable(False)
    log(f"[bench] per-kernel pass: {kreps} steps, {timed_ms:.3f} ms per step")
    return total_ms / steps, per_step, kernels, timed_ms, clk


def run_secondary(w, reps=20, warmup=5, warmup_s=0.05, min_timed_s=0.1):
    """One workload timed launch by launch, per pass (fa_fwd; with a
    backward, fa_bwd after it): untimed launches until at least `warmup` of
    them and `warmup_s` seconds have run (the first tens of milliseconds of a
    burst run while the shader clock is still moving: at N = 8192, D = 128
    the first ~25 ms of launches take ~3% longer than the settled ones), then
    at least `reps` launches and `min_timed_s` seconds, each between the
    events recorded before and after it on the launch stream (mean, median,
    minimum), then as many more between two events only (``batch_ms``: short
    kernels lose a few microseconds to the events between launches).
    Returns a dict with mean, median and minimum per pass and the rates."""
    import statistics

    import torch
    from exact_io_aware_58_amd import fa, inputs

    devs = {n: upload(raw, w.dtype) for n, (_, raw) in inputs.make_inputs(w).items()}
    q, k, v = devs["q"], devs["k"], devs["v"]
    code = {"f32": fa.FA_F32, "bf16": fa.FA_BF16, "f16": fa.FA_F16}[w.dtype]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    args_f = (code, w.B, w.H, w.N, w.D, w.scale, w.causal, q.data_ptr(), k.data_ptr(),
              v.data_ptr(), o.data_ptr(), lse.data_ptr(), sh)

    def fwd():
        rc = fa.fa_fwd(*args_f)
        if rc != fa.FA_OK:
            raise fa.FAError(rc, "fa_fwd")

    def timed(fn):
        # warm-up by count and by time; its last chunk also sizes the timed
        # series (at least `reps` launches and `min_timed_s` seconds)
        done, t0, chunk = 0, time.perf_counter(), max(1, warmup)
        while True:
            c0 = time.perf_counter()
            for _ in range(chunk):
                fn()
            torch.cuda.synchronize()
            done += chunk
            per_launch = (time.perf_counter() - c0) / chunk
            if done >= warmup and time.perf_counter() - t0 >= warmup_s:
                break
            chunk = max(1, min(1000, int(0.01 / max(per_launch, 1e-7))))
        n = max(reps, min(5000, int(min_timed_s / max(per_launch, 1e-7)) + 1))
        # launches enqueued back to back with one event between consecutive
        # launches, so the GPU's queue never waits for the host; then the
        # same number of launches between just two events (no event work
        # between kernels: the rate the kernels sustain when queued)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        counts.append((done, n))
        return per, e0.elapsed_time(e1) / n

    f, b = flops(w)
    out = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "dtype": w.dtype,
           "causal": w.causal, "input_mult": w.input_mult, "min_launches": reps,
           "min_warmup_launches": warmup, "min_warmup_s": warmup_s, "min_timed_s": min_timed_s}
    counts = []  # (warm-up launches, timed launches) per pass

    def summary(res, work):
        t, batch = res
        mean, med, mn = statistics.mean(t), statistics.median(t), min(t)
        return {"ms": mean, "median_ms": med, "min_ms": mn,
                "tflops": work / mean / 1e9, "tflops_median": work / med / 1e9,
                "pct_of_bf16_peak": 100.0 * work / mean / 1e9 / PEAK_BF16_TFLOPS,
                "pct_of_bf16_peak_median": 100.0 * work / med / 1e9 / PEAK_BF16_TFLOPS,
                "batch_ms": batch, "tflops_batch": work / batch / 1e9,
                "pct_of_bf16_peak_batch": 100.0 * work / batch / 1e9 / PEAK_BF16_TFLOPS}

    out["fwd"] = summary(timed(fwd), f)
    if w.backward:
        do = devs["do"]
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        wsb = fa.fa_bwd_workspace_bytes(code, w.B, w.H, w.N, w.D, w.causal)
        ws = torch.empty(wsb, dtype=torch.uint8, device=q.device)
        fwd()
        args_b = (code, w.B, w.H, w.N, w.D, w.scale, w.causal, q.data_ptr(), k.data_ptr(),
                  v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                  dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), wsb, sh)

        def bwd():
            rc = fa.fa_bwd(*args_b)
            if rc != fa.FA_OK:
                raise fa.FAError(rc, "fa_bwd")

        out["bwd"] = summary(timed(bwd), b)
        del dq, dk, dv, ws
    out["fwd"]["warmup_launches"], out["fwd"]["launches"] = counts[0]
    if w.backward:
        out["bwd"]["warmup_launches"], out["bwd"]["launches"] = counts[1]
    log(f"[bench] {w.name}: fwd median {out['fwd']['median_ms']:.4f} ms"
        + (f", bwd median {out['bwd']['median_ms']:.4f} ms" if w.backward else ""))
    del devs, q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def run_split(w, parts, reps=3):
    """The forward of workload `w` assembled from `parts` query blocks and
    `parts` key/value blocks, as `parts` devices holding one block each would
    compute it: every query block attends to each visible key block with
    fa_fwd_partial and folds the results together with fa_merge.  Blocks are
    copied to contiguous buffers before timing (each device would hold its
    own).  Returns the assembled forward's time and rate (credited with the
    whole forward's flops) and the merge kernel's measured bandwidth."""
    import torch
    from exact_io_aware_58_amd import fa, inputs

    devs = {n: upload(raw, w.dtype) for n, (_, raw) in inputs.make_inputs(w).items()
            if n in ("q", "k", "v")}
    code = {"f32": fa.FA_F32, "bf16": fa.FA_BF16, "f16": fa.FA_F16}[w.dtype]
    nb = w.N // parts
    qs, ks, vs = ([devs[n][:, :, i * nb:(i + 1) * nb].contiguous() for i in range(parts)]
                  for n in ("q", "k", "v"))
    del devs
    acc_o = [torch.empty_like(qs[0]) for _ in range(parts)]
    acc_l = [torch.empty((w.B, w.H, nb), dtype=torch.float32, device="cuda") for _ in range(parts)]
    tmp_o, tmp_l = torch.empty_like(qs[0]), torch.empty_like(acc_l[0])
    sh = torch.cuda.current_stream().cuda_stream

    def forward():
        for s_ in range(parts):
            for t in range(parts):
                if w.causal and t > s_:
                    break
                first = t == 0
                o, l = (acc_o[s_], acc_l[s_]) if first else (tmp_o, tmp_l)
                rc = fa.fa_fwd_partial(code, w.B, w.H, nb, nb, w.D, w.scale, w.causal,
                                       s_ * nb, t * nb, qs[s_].data_ptr(), ks[t].data_ptr(),
                                       vs[t].data_ptr(), o.data_ptr(), l.data_ptr(), sh)
                if rc != fa.FA_OK:
                    raise fa.FAError(rc, "fa_fwd_partial")
                if not first:
                    rc = fa.fa_merge(code, w.B, w.H, nb, w.D, acc_o[s_].data_ptr(),
                                     acc_l[s_].data_ptr(), tmp_o.data_ptr(), tmp_l.data_ptr(), sh)
                    if rc != fa.FA_OK:
                        raise fa.FAError(rc, "fa_merge")

    forward()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fa.fa_timing_enable(True)
    e0.record()
    for _ in range(reps):
        forward()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n, mms, _ = fa.fa_timing_read(fa.FA_KERNEL_MERGE)
    fa.fa_timing_enable(False)
    f, _ = flops(w)
    sub = type(w)(w.name, w.seed, w.B, w.H, nb, w.D, w.dtype, w.causal, False)
    _, merge_bytes = kernel_algorithmic(sub)["merge"]
    merge_ms = mms / n if n else None
    return {
        "workload": f"{w.name} forward from {parts} query x {parts} key blocks",
        "ms": ms, "tflops": f / (ms / 1e3) / 1e12,
        "merge": {"launches_per_forward": n // reps if n else 0, "avg_ms": merge_ms,
                  "GB/s": merge_bytes / (merge_ms / 1e3) / 1e9 if merge_ms else None,
                  "frac_of_hbm_peak": (merge_bytes / (merge_ms / 1e3) / 1e9 / PEAK_HBM_GBS)
                  if merge_ms else None},
    }


def blas_info():
    """(vendor and version of the BLAS numpy calls, threads it uses)."""
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        pools = []
    if not pools:
        return "unknown", 1
    p = pools[0]
    return f"{p.get('internal_api', '?')} {p.get('version', '')}".strip(), int(p.get("num_threads", 1))


def cpu_baseline(w, rows):
    """The float64 oracle on the leading rows x rows block of head 0 (causal:
    those queries see only those keys, so the block is a self-contained slice
    of the workload), forward + backward, with the BLAS thread pool set to
    the CPUs this process may run on.  Also reports the whole workload's
    oracle time extrapolated by flops from the sample (labelled as such)."""
    import numpy as np
    import oracle
    from exact_io_aware_58_amd import inputs
    affinity = len(os.sched_getaffinity(0))
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=affinity, user_api="blas")
    except Exception:  # pragma: no cover
        pass
    vendor, threads = blas_info()
    rows = min(rows, w.N)
    t = {}
    for name in ("q", "k", "v", "do"):
        x, _ = inputs.draw(w.seed, name, w.shape, w.dtype, w.input_mult if name != "do" else 1.0)
        t[name] = x[:1, :1, :rows].astype(np.float64)
    log(f"[bench] cpu baseline: oracle on head 0, rows [0, {rows}), {threads} BLAS threads "
        f"({vendor}) ...")
    t0 = time.perf_counter()
    oracle.attention_fwd(t["q"], t["k"], t["v"], w.scale, w.causal)
    if w.backward:
        oracle.attention_bwd(t["q"], t["k"], t["v"], t["do"], w.scale, w.causal)
    sec = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    sub = type(w)(w.name, w.seed, 1, 1, rows, w.D, w.dtype, w.causal, w.backward)
    f, b = flops(sub)
    fw, bw = flops(w)
    return {
        "value": (f + b) / sec / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"head 0 of batch 0, leading {rows}x{rows} "
                  f"{'causal ' if w.causal else ''}block, "
                  f"{'fwd+bwd' if w.backward else 'fwd'} in float64 ({sec:.1f} s)",
        "seconds": sec,
        "affinity_cpus": affinity,
        "blas": vendor,
        "extrapolated_full_workload_s": sec * (fw + bw) / (f + b),
        "extrapolation": "sample seconds x (workload flops / sample flops); not measured",
    }


def three_kernel_forward(q, k, v, scale):
    """The unfused attention forward in PyTorch on the same GPU: scores and
    probabilities materialised in HBM between a matmul, a softmax and a
    matmul (plus the copy that makes K^T contiguous and the scaling)."""
    import torch
    s_ = torch.matmul(q, k.transpose(-2, -1).contiguous()) * scale
    p_ = torch.softmax(s_, dim=-1)
    return torch.matmul(p_, v)


def run_io(ns, heads=16, D=64, passes=2):
    """HBM bytes of one forward pass, fused against the three-kernel path,
    for counting under `rocprofv3 --pmc FETCH_SIZE` (then `WRITE_SIZE`): per
    N, once the inputs are resident, `passes` times the fused forward and then
    the three-kernel forward, each followed by a synchronisation, and nothing
    else on the GPU in between.  B = 1, bf16, no mask.  Prints one JSON line
    per N with the kernels' wall times (each pass timed alone)."""
    import torch
    from exact_io_aware_58_amd import fa, inputs

    scale = 1.0 / D ** 0.5
    for N in ns:
        w = inputs.Workload(f"io_n{N}", 7, 1, heads, N, D, "bf16", False, False)
        devs = {n: upload(raw, "bf16") for n, (_, raw) in inputs.make_inputs(w).items()}
        q, k, v = devs["q"], devs["k"], devs["v"]
        torch.cuda.synchronize()
        row = {"N": N, "B": 1, "H": heads, "D": D, "causal": False, "passes": passes,
               "fused_ms": [], "three_kernel_ms": []}
        for _ in range(passes):
            for key, fn in (("fused_ms", lambda: fa.forward(q, k, v, scale, False)),
                            ("three_kernel_ms", lambda: three_kernel_forward(q, k, v, scale))):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                out = fn()
                e1.record()
                torch.cuda.synchronize()
                row[key].append(e0.elapsed_time(e1))
                del out
        print(json.dumps(row), flush=True)
        del q, k, v, devs
        torch.cuda.empty_cache()


def run_sweep(ns, heads=16, D=64, reps=5):
    """Sequence-length sweep (one JSON line per N): forward and backward time
    and device memory of this library beside the three-kernel PyTorch path
    (matmul, softmax, matmul on the same GPU, bf16, non-causal), which
    materialises the N x N scores and probabilities in HBM.  The reference
    path runs forward only (its autograd backward issues batched bf16
    products on transposed views, which are not run on this GPU)."""
    import numpy as np
    import torch
    from exact_io_aware_58_amd import fa, inputs

    scale = 1.0 / D ** 0.5
    for N in ns:
        w = inputs.Workload(f"sweep_n{N}", 7, 1, heads, N, D, "bf16", False, True)
        devs = {n: upload(raw, "bf16") for n, (_, raw) in inputs.make_inputs(w).items()}
        q, k, v, do = devs["q"], devs["k"], devs["v"], devs["do"]
        f, b = flops(w)
        row = {"N": N, "B": 1, "H": heads, "D": D, "causal": False}

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        o, lse = fa.forward(q, k, v, scale, False)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, False)
        torch.cuda.synchronize()
        row["fa_extra_bytes"] = torch.cuda.max_memory_allocated() - base
        ws = torch.empty(fa.workspace_bytes(q), dtype=torch.uint8, device=q.device)
        row["fa_fwd_ms"] = timed(lambda: fa.forward(q, k, v, scale, False, out=o, lse=lse))
        row["fa_bwd_ms"] = timed(lambda: fa.backward(q, k, v, o, do, lse, scale, False, dq=dq,
                                                     dk=dk, dv=dv, workspace=ws))
        row["fa_fwd_tflops"] = f / row["fa_fwd_ms"] / 1e9
        row["fa_bwd_tflops"] = b / row["fa_bwd_ms"] / 1e9
        del dq, dk, dv, ws

        def naive():
            return three_kernel_forward(q, k, v, scale)

        try:
            torch.cuda.synchronize()
            base = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            ref = naive()
            torch.cuda.synchronize()
            row["naive_extra_bytes"] = torch.cuda.max_memory_allocated() - base
            row["naive_max_abs_diff"] = float((ref.float() - o.float()).abs().max())
            del ref
            row["naive_fwd_ms"] = timed(naive)
            row["fwd_speedup"] = row["naive_fwd_ms"] / row["fa_fwd_ms"]
        except torch.cuda.OutOfMemoryError:
            row["naive_fwd_ms"] = "out of memory"
        torch.cuda.empty_cache()
        print(json.dumps(row), flush=True)
        del q, k, v, do, o, lse, devs
        torch.cuda.empty_cache()


def run_update_probe(mib=256, passes=8, reps=3, mfma_s=2.5):
    """Rate of fp32 updates to device memory (plain store, plain
    read-modify-write, fp32 atomic add), from the probe library built beside
    libfa.so: each pass updates every float of a `mib` MiB buffer once, one
    lane per element, 256 contiguous bytes per wave.  The atomic adds are
    checked (every element ends at passes x launches).  Prints one JSON line:
    the best of `reps` timed launches per mode, as GB/s of 4-byte updates.
    Then the register-only bf16 MFMA rate over `mfma_s` seconds of launches,
    with the shader clock sampled meanwhile (a second JSON line)."""
    import ctypes

    import torch
    from exact_io_aware_58_amd import build

    if not os.path.exists(build.PROBE_LIB):
        raise RuntimeError(f"{build.PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.fa_probe_update.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.fa_probe_update.restype = ctypes.c_int
    n = mib * (1 << 20) // 4
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    row = {"probe": "fp32 updates", "buffer_mib": mib, "passes_per_launch": passes,
           "unit": "GB/s of 4-byte updates"}
    for mode, name in ((0, "store"), (1, "read_modify_write"), (2, "atomic_add")):
        buf.zero_()
        launches = 0
        best = None
        for r in range(reps + 1):  # the first launch is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.fa_probe_update(mode, buf.data_ptr(), n, passes, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"fa_probe_update({mode}) returned {rc}")
            launches += 1
            if r > 0:
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
        row[name] = n * 4 * passes / (best / 1e3) / 1e9
        if mode == 2:
            row["atomic_add_checked"] = bool((buf == float(passes * launches)).all().item())
    print(json.dumps(row), flush=True)
    del buf

    # Register-only bf16 MFMA loop: 8 four-wave workgroups per CU, launches
    # back to back for `mfma_s` seconds with the shader clock sampled.
    lib.fa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_mfma.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus * 8, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 16

    def launch():
        rc = lib.fa_probe_mfma(out.data_ptr(), blocks, iters, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"fa_probe_mfma returned {rc}")

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(20):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 20
    count = max(20, int(mfma_s * 1e3 / per))
    clock = ClockSampler()
    t0 = time.perf_counter()
    clock.start()
    e0.record(stream)
    for _ in range(count):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    clock.stop()
    window = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / count
    tflops = flops / (ms / 1e3) / 1e12
    mfma = {"probe": "register-only bf16 MFMA (32x32x16, 4 independent chains per wave)",
            "workgroups": blocks, "waves_per_cu": 32, "launches": count, "ms_per_launch": ms,
            "tflops": tflops, "pct_of_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
            "sclk": clock.summary(window)}
    if mfma["sclk"]:
        peak_clk = PEAK_BF16_TFLOPS * mfma["sclk"]["mean_mhz"] / NOMINAL_SCLK_MHZ
        mfma["peak_at_measured_clock"] = peak_clk
        mfma["pct_of_peak_at_measured_clock"] = 100.0 * tflops / peak_clk
    print(json.dumps(mfma), flush=True)


def copy_calibration(mib):
    """One plain device copy of `mib` MiB (read and written once): a kernel of
    known size against which HBM byte counters are scaled."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {mib} MiB read + {mib} MiB written")
    del src, dst


class ClockSampler:
    """Shader clock while the GPU runs the workload, from the AMD SMI
    library's copy of the driver's metrics table (current clock of each XCD,
    averaged over the XCDs).  The table refreshes about once a second, so a
    thread polls it every 10 ms between start() and stop() and keeps one
    sample per refresh, dropping the table current at start() and the first
    refresh after it (which may still cover time before the window).  It
    makes no HIP call.  summary() is None without the library or samples."""

    def __init__(self, period=0.01):
        import threading
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                self._smi, self._handle = amdsmi, handles[0]
        except Exception as e:  # pragma: no cover - depends on the box
            log(f"[bench] no shader-clock samples: {e}")

    def read(self):
        """(refresh counter, mean current clock over the XCDs in MHz) or None."""
        try:
            m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        except Exception:  # pragma: no cover
            return None
        vals = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float)) and v > 0]
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [m["current_gfxclk"]]
        stamp = m.get("system_clock_counter")
        return (stamp, sum(vals) / len(vals)) if vals and stamp is not None else None

    def _run(self, first):
        seen = {first}
        fresh = 0
        while not self._stop.is_set():
            r = self.read()
            if r is not None and r[0] not in seen:
                seen.add(r[0])
                fresh += 1
                if fresh > 1:
                    self.samples.append(r[1])
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._handle is None:
            return
        r = self.read()
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, args=(r[0] if r else None,),
                                        daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self, window_s):
        if not self.samples:
            return None
        import statistics
        return {"source": "AMD SMI metrics table (current clock per XCD, averaged), one sample "
                          "per table refresh while the workload's steps ran back to back",
                "window_s": window_s, "samples": len(self.samples),
                "mean_mhz": statistics.mean(self.samples),
                "min_mhz": min(self.samples), "max_mhz": max(self.samples)}


NOMINAL_SCLK_MHZ = 2400.0

SECONDARY = ("c2", "c3", "n4k_d128", "n8k_d128", "c4", "train_d128")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", help="c1..c5 (default c5)")
    ap.add_argument("--cpu-rows", type=int, default=32768,
                    help="rows of the oracle sample timed for cpu_baseline (0: skip)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary workloads (c2, c3, D=128 forwards at N=4096, "
                         "8192, 16384, the D=128 training step) and the block-split forward")
    ap.add_argument("--clock-window", type=float, default=3.5,
                    help="seconds of extra steps (outside the timed regions) during which the "
                         "shader clock is sampled (0: skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a "
                         "known-size kernel for scaling HBM byte counters)")
    ap.add_argument("--sweep", default="",
                    help="comma-separated sequence lengths: print one JSON line per N "
                         "comparing with the three-kernel PyTorch path instead of the bench line")
    ap.add_argument("--sweep-d", type=int, default=64, choices=(64, 128),
                    help="head dimension of the --sweep and --io runs (B=1, H=16)")
    ap.add_argument("--io", default="",
                    help="comma-separated sequence lengths: run the fused and the "
                         "three-kernel forward twice each per N and nothing else, for "
                         "counting HBM bytes under rocprofv3 --pmc")
    ap.add_argument("--probe", action="store_true",
                    help="rate of fp32 stores, read-modify-writes and atomic adds to "
                         "device memory (the probe library), then exit")
    args = ap.parse_args()
    if args.probe:
        run_update_probe()
        return
    if args.sweep:
        run_sweep([int(x) for x in args.sweep.split(",")], D=args.sweep_d)
        return
    if args.io:
        run_io([int(x) for x in args.io.split(",")], D=args.sweep_d)
        if args.copy_mib > 0:
            copy_calibration(args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path is built and timed on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import statistics

    from exact_io_aware_58_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    clock = ClockSampler()
    ms, per_step, kernels, kernel_pass_ms, clk = run_gpu(w, args.steps, args.warmup, clock,
                                                         args.clock_window)
    f, b = flops(w)
    value = (f + b) / (ms / 1e3) / 1e12
    med, mn = statistics.median(per_step), min(per_step)

    alg = kernel_algorithmic(w)
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    bound, work = alg[dom]
    dur = kernels[dom]["avg_ms"] / 1e3
    if bound == "mfma":
        achieved, peak, unit = work / dur / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / dur / 1e9, PEAK_HBM_GBS, "GB/s"
    for name, kv in kernels.items():
        kb, kw = alg[name]
        kv["achieved"] = kw / (kv["avg_ms"] / 1e3) / (1e12 if kb == "mfma" else 1e9)
        kv["unit"] = "TFLOP/s" if kb == "mfma" else "GB/s"

    passes = {}
    if "fwd" in kernels:
        passes["fwd"] = {"ms": kernels["fwd"]["avg_ms"],
                         "tflops": f / (kernels["fwd"]["avg_ms"] / 1e3) / 1e12}
    if w.backward:
        bms = sum(kernels[k]["avg_ms"] for k in ("bwd_delta", "bwd_dkdv", "bwd_dq", "bwd_dkdv_dq")
                  if k in kernels)
        passes["bwd"] = {"ms": bms, "tflops": b / (bms / 1e3) / 1e12}
    for p in passes.values():
        p["pct_of_bf16_peak"] = 100.0 * p["tflops"] / PEAK_BF16_TFLOPS

    roofline = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak,
                "unit": unit, "frac": achieved / peak,
                "traffic": profiled_traffic(w.name, dom)}
    if clk and bound == "mfma":
        # the same peak scaled to the shader clock sampled while the steps ran
        roofline["peak_at_measured_clock"] = peak * clk["mean_mhz"] / NOMINAL_SCLK_MHZ
        roofline["frac_at_measured_clock"] = achieved / roofline["peak_at_measured_clock"]

    secondary = {}
    if not args.no_secondary:
        for key in SECONDARY:
            if key == args.workload:
                continue
            sw = inputs.WORKLOADS[key]
            secondary[sw.name] = run_secondary(sw, reps=max(20, args.steps),
                                               warmup=max(5, args.warmup))

    split = None
    if not args.no_secondary and w.N % 4 == 0:
        split = run_split(w, 4)
        log(f"[bench] split forward: {split['ms']:.3f} ms")

    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)

    cpu = cpu_baseline(w, args.cpu_rows) if args.cpu_rows > 0 else None

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "causal": w.causal, "passes": "fwd+bwd" if w.backward else "fwd",
                   "flops_per_step": f + b},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "step_ms": {"mean": ms, "median": med, "min": mn, "steps": len(per_step),
                    "tflops_median": (f + b) / med / 1e9, "tflops_min_time": (f + b) / mn / 1e9},
        "sclk": clk,
        "pct_of_bf16_peak_at_measured_clock": (
            100.0 * value / (PEAK_BF16_TFLOPS * clk["mean_mhz"] / NOMINAL_SCLK_MHZ)
            if clk else None),
        "passes": passes,
        "kernels": kernels,
        "kernel_timing_pass": {"steps": max(args.steps, 3), "ms_per_step": kernel_pass_ms,
                               "note": "per-kernel events on; separate from the headline steps"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if secondary:
        out["secondary"] = secondary
    if split:
        out["split_fwd"] = split
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
