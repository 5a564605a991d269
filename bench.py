#!/usr/bin/env python3
"""Benchmark of the attention op's hot path on one MI355X.

One step is one decode step of the Llama-3-8B-shaped GQA workload (T=1,
S=32768, heads 32, kvHeads 8, headDim 128, causal, posOffset 32767): the
new K and V rows are appended at row 32767 and attention runs over the
whole cache, in one call (attn_forward_append: decode_split reads the new
rows from their buffers, stores them into the caches and attends over them
with the rest; then combine). The same step made of separate calls
(attn_cache_write2, then attn_forward) is timed too. K/V
caches rotate over two copies (512 MiB together) so no step finds its
working set in the 256 MB Infinity Cache.

The prefill is measured first, so the decode's warm-up steps start on a GPU
whose clocks are already up (timed right after start-up, the decode kernel
measured about 1 us slower over its first few hundred launches).

`value` is the decode's algorithmic KV bandwidth: the bytes attention must
move (every visible K and V row once, plus q and out) per step time, in
GB/s. `roofline` rates the dominant kernel, decode_split, on its own: the
same algorithmic bytes over its average duration, timed with HIP events
that each launch's dispatch stamps on the stream it runs on, against the
8 TB/s HBM peak. `cpu_baseline` times the CPU oracle on the same inputs.

The same line carries `prefill`: the Llama-3-8B-shaped causal prefill
(T=S=4096), whose algorithmic flops (heads x visible (query, key) pairs x
(2 headDim + 2 vHeadDim)) over the call time give TFLOP/s, rated against the
157.3 TFLOP/s fp32 matrix peak.

`rope` holds the rotary embedding: the same decode step with rope fused in
(the new K row rotated into a staging row, then attn_forward_append with q
rotated as attention loads it; also timed as three separate calls) and the
standalone rope kernel on a prefill-sized q, rated against HBM.

`configs` lists the other workloads the same way (their own plan, kernel
time, call rate, roofline and sampled-row parity): the Llama-shaped chunked
prefill (T=512 at posOffset 3584), the Gemma-2-shaped sliding-window prefill
(T=S=8192, headDim 256, softcap 50, window 4096), and the latent-shaped
ALiBi + per-head bias decode (S=8192, headDim 192, vHeadDim 128) and
non-causal prefill (T=S=1024), and the Llama-shaped streaming decode (window
4096 plus 4 attention sinks over a 32768-row cache), the wide-group decodes
(Llama-3-70B-shaped 64 heads over 8 KV heads, Qwen2-7B-shaped 28 over 4),
and the Llama-shaped decode with a T5-style bucketed position bias or with
relative key/value embeddings.

`mla` holds latent (MLA) attention in absorbed form: the DeepSeek-V2-Lite-
shaped decode (16 heads, kv_rank 512, S=8192) and a DeepSeek-V3-shaped one
(128 heads, S=32768): call time, the three kernels' durations, and the
split kernel's roofline (HBM or fp32 matrix peak, whichever bounds it).

Every benchmarked output is checked against the CPU oracle on the same
inputs, every row of it (the prefill-shaped ones too, which takes the oracle
tens of seconds for the largest; --sampled-parity checks ~30 rows instead).

`--only NAME,...` times just the named workloads of workloads.py (or ROPE,
the rope section; one record each, no headline line), after one plain
134,213,632-byte copy that calibrates the profiler's traffic counters: the
profiles under profiles/ run the profiler over one workload at a time this way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--prefill-steps K] [--no-configs] [--sampled-parity] [--only NAME,...]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV GB/s + prefill TFLOP/s (f32), % of MI355X roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources a kernel's counters depend on: its own files, and the planner
# (attn_api.hip), which sets its grid, split counts and workspace layout.
KERNEL_SOURCES = {
    "decode_split": ["gqa_scaled_dot_amd/csrc/decode.hip", "gqa_scaled_dot_amd/csrc/device_common.h",
                     "gqa_scaled_dot_amd/csrc/kernels.h", "gqa_scaled_dot_amd/csrc/rope_device.h"],
    "prefill": ["gqa_scaled_dot_amd/csrc/prefill.hip", "gqa_scaled_dot_amd/csrc/prefill16.hip",
                "gqa_scaled_dot_amd/csrc/prefill_common.h", "gqa_scaled_dot_amd/csrc/device_common.h",
                "gqa_scaled_dot_amd/csrc/kernels.h", "gqa_scaled_dot_amd/csrc/rope_device.h"],
    "rope": ["gqa_scaled_dot_amd/csrc/rope.hip", "gqa_scaled_dot_amd/csrc/rope_device.h",
             "gqa_scaled_dot_amd/csrc/kernels.h"],
    "decode_mfma": ["gqa_scaled_dot_amd/csrc/decode_mfma.hip", "gqa_scaled_dot_amd/csrc/device_common.h",
                    "gqa_scaled_dot_amd/csrc/kernels.h", "gqa_scaled_dot_amd/csrc/rope_device.h"],
    "mla_split": ["gqa_scaled_dot_amd/csrc/mla.hip", "gqa_scaled_dot_amd/csrc/device_common.h",
                  "gqa_scaled_dot_amd/csrc/kernels.h"],
}
for _srcs in KERNEL_SOURCES.values():
    _srcs.append("gqa_scaled_dot_amd/csrc/attn_api.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from rocprofv3 counters
    (profiles/traffic.json), if they were taken on this very kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f).get("entries", [])
    except (OSError, ValueError):
        return None
    for rec in entries:
        if rec.get("kernel") == kernel and rec.get("workload") == workload:
            return rec.get("bytes_per_launch") if rec.get("source_sha256") == source_hash(kernel) else None
    return None


def decode_algorithmic_bytes(w) -> int:
    """Every visible K and V row once (window rows and the sinks below them),
    plus q, out and the visible bias entries."""
    lo = max(0, w.posOffset - (w.window or 0) + 1) if w.window else 0
    hi = min(w.S, w.posOffset + w.T)
    rows = hi - lo
    if w.window and w.sinks:
        rows += min(w.sinks, lo)
    b = rows * w.G * (w.headDim + w.Dv) * 4
    b += w.T * w.heads * w.headDim * 4 + w.T * w.heads * w.Dv * 4
    if w.bias == "HTS":
        b += w.heads * w.T * rows * 4
    elif w.bias == "TS":
        b += w.T * rows * 4
    return b


def visible_pairs(w) -> int:
    """Visible (query, key) pairs of one head under the causal/window rule."""
    import numpy as np
    pos = (w.posOffset or 0) + np.arange(w.T, dtype=np.int64)
    if w.causal:
        hi = np.minimum(pos, w.S - 1)
        lo = np.maximum(0, pos - w.window + 1) if w.window else np.zeros_like(pos)
    else:
        hi = np.minimum(pos + w.window, w.S - 1) if w.window else np.full_like(pos, w.S - 1)
        lo = np.maximum(0, pos - w.window) if w.window else np.zeros_like(pos)
    return int(np.maximum(hi - lo + 1, 0).sum())


def host_cpu() -> str:
    """The host CPU's model name (the oracle's hardware), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_clocks():
    """Current shader and memory clock of the GPU, read from the amdgpu driver's
    sysfs files (the ones rocm-smi reads: the level marked '*'), or None where
    they are absent or more than one card shows them."""
    import glob
    cards = sorted(glob.glob("/sys/class/drm/card[0-9]*/device/pp_dpm_sclk"))
    if len(cards) != 1:
        return None
    dev = os.path.dirname(cards[0])
    out = {}
    for name in ("sclk", "mclk", "fclk"):
        try:
            with open(os.path.join(dev, "pp_dpm_" + name)) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        out[name] = line.split(":", 1)[1].replace("*", "").strip()
        except OSError:
            pass
    return out or None


def affinity_cpus() -> int:
    """CPUs this process may run on (len(os.sched_getaffinity(0)))."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# A one-GPU machine grants its jobs 16 host CPUs, whatever the affinity mask
# shows, so the oracle runs at most 16 threads; the records state both counts.
CPU_SHARE = 16


def cpu_threads() -> int:
    return max(1, min(affinity_cpus(), CPU_SHARE))


CALIBRATION_COPY_BYTES = 32767 * 4096  # the Llama-shaped decode's cache fill: 32767 rows of 4 KiB, 134,213,632 bytes


def calibration_copy():
    """One plain copy of known size (attn_cache_write of 32767 rows x 4 KiB,
    the Llama-shaped decode's cache fill): the reference that scales the
    profiler's FETCH_SIZE / WRITE_SIZE readings to bytes in every counter pass."""
    import torch

    import gqa_scaled_dot_amd as ga
    src = torch.zeros((32767, 1024), dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ga.attn_cache_write(dst, src, 0)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def run_decode(args):
    import numpy as np
    import torch

    import gqa_scaled_dot_amd as ga
    import workloads

    w = workloads.LLAMA_DECODE
    params = w.params()
    dev = torch.device("cuda:0")
    q, k, v, _ = w.tensors()
    log(f"[bench] workload: {w.name}")
    plan = ga.attn_plan(w.T, w.S, **params)
    log(f"[bench] plan: {plan}")

    n_buf = 2
    qd = torch.from_numpy(q).to(dev)
    kd = torch.from_numpy(k).to(dev)
    vd = torch.from_numpy(v).to(dev)
    kc = [torch.empty_like(kd) for _ in range(n_buf)]
    vc = [torch.empty_like(vd) for _ in range(n_buf)]
    for b in range(n_buf):  # the past rows, through cache_write
        ga.attn_cache_write(kc[b], kd[:w.S - 1], 0)
        ga.attn_cache_write(vc[b], vd[:w.S - 1], 0)
    new_k, new_v = kd[w.S - 1:], vd[w.S - 1:]
    del kd, vd
    out = torch.empty((w.T, w.heads * w.Dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ga.attn_workspace_size(w.T, w.S, **params), 256), dtype=torch.uint8, device=dev)

    steps = [ga.prepare_forward_append(qd, kc[b], vc[b], new_k, new_v, w.S - 1, out=out, workspace=ws, **params)
             for b in range(n_buf)]
    separate = [(ga.prepare_cache_write2(kc[b], new_k, vc[b], new_v, w.S - 1),
                 ga.prepare_forward(qd, kc[b], vc[b], out=out, workspace=ws, **params)) for b in range(n_buf)]

    def step(i):
        steps[i % n_buf]()

    def step_separate(i):
        append, attend = separate[i % n_buf]
        append()
        attend()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps between two events on the stream the kernels run on.
    ga.attn_timing_enable(True)
    for name in ("decode_split", "combine", "cache_write"):
        ga.attn_timing_collect(name)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    clocks = device_clocks()  # right after the timed steps, while the clocks are still up
    ms_timed = e0.elapsed_time(e1) / args.steps
    split_ms, split_n = ga.attn_timing_collect("decode_split")
    comb_ms, comb_n = ga.attn_timing_collect("combine")
    cw_ms, cw_n = ga.attn_timing_collect("cache_write")
    ga.attn_timing_enable(False)

    # The same loop without per-kernel events, for the step time itself.
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    # The same step as separate calls, for comparison (after its own warm-up).
    for i in range(args.warmup):
        step_separate(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step_separate(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_separate = e0.elapsed_time(e1) / args.steps
    for i in range(2):  # leave `out` as the fused step computes it
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] step {ms_per_step * 1e3:.2f} us (with kernel events {ms_timed * 1e3:.2f} us; "
        f"as separate calls {ms_separate * 1e3:.2f} us); "
        f"decode_split {split_ms / max(split_n, 1) * 1e3:.2f} us x{split_n}, "
        f"combine {comb_ms / max(comb_n, 1) * 1e3:.2f} us x{comb_n}, "
        f"cache_write {cw_ms / max(cw_n, 1) * 1e3:.2f} us x{cw_n}")

    alg_bytes = decode_algorithmic_bytes(w)
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    split_avg_s = split_ms / split_n * 1e-3
    achieved = alg_bytes / split_avg_s / 1e9
    traffic = measured_traffic("decode_split", w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "decode_split", "bytes_per_launch": alg_bytes,
                "avg_launch_us": round(split_avg_s * 1e6, 3)}

    # Parity of the benchmarked output against the oracle (same seeded inputs).
    import oracle
    threads = cpu_threads()
    got = out.cpu().numpy().astype(np.float64)
    cpu_baseline = None
    t0 = time.perf_counter()
    ref = oracle.attention(q, k, v, threads=threads, **params)
    t_one = time.perf_counter() - t0
    err = np.abs(got - ref)
    parity_ok = bool(np.all(err <= 1e-4 + 1e-4 * np.abs(ref)))
    log(f"[bench] parity vs oracle: max |err| {err.max():.3e} ok={parity_ok}")
    if not args.no_cpu:
        reps, total = 1, t_one
        budget = 10.0
        while total < budget and reps < 1000:
            t0 = time.perf_counter()
            oracle.attention(q, k, v, threads=threads, **params)
            total += time.perf_counter() - t0
            reps += 1
        cpu_baseline = {"value": round(alg_bytes * reps / total / 1e9, 4), "unit": "GB/s",
                        "cores": threads, "affinity_cpus": affinity_cpus(), "kind": "oracle", "cpu": host_cpu(),
                        "sample": f"the full decode step (1 query row, 32 heads, 32768 keys), "
                                  f"{reps} runs in {total:.1f} s, f64"}

    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "S": w.S, "heads": w.heads, "kvHeads": w.G,
                   "headDim": w.headDim, "vHeadDim": w.Dv, "posOffset": w.posOffset,
                   "causal": True, "kv_buffers": n_buf, "splits": plan["splits"],
                   "step": "attn_forward_append: the new K and V rows written and attended in decode_split "
                           "(one more split per KV head), then combine"},
        "ms_per_step_separate_calls": round(ms_separate, 6),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity": {"max_abs_err": float(err.max()), "ok": parity_ok},
        "device": {"clocks_after_timed_steps": clocks, "host_cpu": host_cpu(), "host_threads": threads,
                   "host_affinity_cpus": affinity_cpus(),
                   "host_threads_note": f"the oracle runs min(affinity CPUs, {CPU_SHARE}) threads: "
                                        f"a one-GPU box grants {CPU_SHARE} host CPUs"},
    }


def sampled_rows(w, n_random=24):
    """Rows whose outputs the oracle checks: both ends, the middle, seeded random ones."""
    import numpy as np
    fixed = [0, 1, 2, 31, 32, w.T // 2 - 1, w.T // 2, w.T - 2, w.T - 1]
    rnd = np.random.default_rng(7).integers(0, w.T, n_random) if w.T > 1 else []
    return sorted(set(r for r in fixed + [int(x) for x in rnd] if 0 <= r < w.T))


def relpos_terms(w, kind):
    """Host tables of a relative-position term for workload w: a T5-style
    bucketed bias (32 buckets, the log-spaced thresholds T5's bucket function
    gives for max distance 128) or relative key/value embeddings (max
    distance 128)."""
    import math
    import numpy as np
    import workloads as wl
    if kind == "position_bias":
        th, prev = [], -1
        for d in range(4096):  # first distance of each unidirectional T5 bucket
            b = d if d < 16 else min(16 + int(math.log(d / 16) / math.log(128 / 16) * 16), 31)
            if b != prev:
                th.append(d)
                prev = b
        return {"position_bias": {"weight": wl.normal((len(th), w.heads), 31, 3), "buckets": th}}
    m = 128
    return {"relative_kv": {"key": wl.normal((2 * m + 1, w.headDim), 32, 1),
                            "value": wl.normal((2 * m + 1, w.Dv), 32, 2), "max_distance": m}}


def _device_terms(extra, dev):
    """The same terms with their tables on the GPU (for the library)."""
    import torch
    out = {}
    for key, term in extra.items():
        out[key] = {k: (torch.from_numpy(v).to(dev) if hasattr(v, "dtype") else v) for k, v in term.items()}
    return out


def run_config(w, args, kv_buffers=1, extra=None, label=None):
    """Time attn_forward on one workload: kernel durations from dispatch-stamped
    events, the call time from a plain loop; the result checked against the
    oracle on sampled rows. Decode-shaped plans are rated in GB/s against HBM,
    prefill-shaped ones in TFLOP/s against the fp32 matrix peak."""
    import numpy as np
    import torch

    import gqa_scaled_dot_amd as ga
    import oracle

    dev = torch.device("cuda:0")
    extra = extra or {}
    params = dict(w.params(), **_device_terms(extra, dev))
    q, k, v, bias = w.tensors()
    kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    plan = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)
    name = label or w.name
    log(f"[bench] workload: {name}; plan {plan}")
    main_kernel = {"decode": "decode_mfma" if plan["variant"] == 1 else "decode_split",
                   "prefill": "prefill"}.get(plan["path"], "generic")
    qd = torch.from_numpy(q).to(dev)
    # Several copies of the K/V (and bias) so a timed call does not find them
    # in the 256 MB MALL: decode plans rotate over at least 512 MiB of reads.
    if plan["path"] == "decode":
        kv_buffers = min(16, max(kv_buffers, -(-(512 << 20) // decode_algorithmic_bytes(w))))
    kv = [tuple(torch.from_numpy(x).to(dev) if x is not None else None for x in (k, v, bias))
          for _ in range(kv_buffers)]
    out = torch.empty((w.T, w.heads * w.Dv), dtype=torch.float32, device=dev)
    ws_bytes = ga.attn_workspace_size(w.T, w.S, bias_kind=kind, **params)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    calls = [ga.prepare_forward(qd, kb, vb, bb, out=out, workspace=ws, **params) for kb, vb, bb in kv]
    n = args.prefill_steps if plan["path"] != "decode" else args.steps
    for i in range(max(2, args.warmup // 5)):
        calls[i % kv_buffers]()
    torch.cuda.synchronize()
    # Kernel durations from dispatch-stamped events ...
    ga.attn_timing_enable(True)
    for kname in (main_kernel, "combine", "prefill_band"):
        ga.attn_timing_collect(kname)
    for i in range(n):
        calls[i % kv_buffers]()
    torch.cuda.synchronize()
    k_ms, k_n = ga.attn_timing_collect(main_kernel)
    c_ms, c_n = ga.attn_timing_collect("combine")
    # Relative embeddings at 128-wide heads: the band tiles' launch counts
    # with the prefill kernel's.
    b_ms, b_n = ga.attn_timing_collect("prefill_band")
    ga.attn_timing_enable(False)
    # ... and the call time from a loop without them.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        calls[i % kv_buffers]()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / n
    kern_s = k_ms / k_n * 1e-3 + (b_ms / b_n * 1e-3 if b_n else 0.0)
    if plan["path"] == "decode":
        work = decode_algorithmic_bytes(w)
        achieved, value, unit, peak, bound = work / kern_s / 1e9, work / (ms_call * 1e-3) / 1e9, \
            "GB/s", HBM_PEAK_GBS, "hbm"
    else:
        work = w.heads * visible_pairs(w) * (2 * w.headDim + 2 * w.Dv)
        achieved, value, unit, peak, bound = work / kern_s / 1e12, work / (ms_call * 1e-3) / 1e12, \
            "TFLOP/s", FP32_PEAK_TFLOPS, "mfma"
    log(f"[bench]   call {ms_call * 1e3:.1f} us, {main_kernel} {kern_s * 1e6:.1f} us x{k_n}"
        + (f" (band launch {b_ms / b_n * 1e3:.1f} us of it)" if b_n else "")
        + (f", combine {c_ms / c_n * 1e3:.2f} us" if c_n else "")
        + f": {achieved:.2f} {unit} = {achieved / peak:.1%} of {peak}")
    # The oracle checks every output row (prefill-shaped calls too, unless
    # --sampled-parity asks for a row sample).
    rows = sampled_rows(w) if (args.sampled_parity and w.T > 1) else None
    t_oracle = time.perf_counter()
    ref = oracle.attention(q, k, v, bias, rows=rows, threads=cpu_threads(), **w.params(), **extra)
    t_oracle = time.perf_counter() - t_oracle
    got = out.cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    err = np.abs(got - ref)
    ok = bool(np.all(err <= 1e-4 + 1e-4 * np.abs(ref)))
    n_rows = w.T if rows is None else len(rows)
    log(f"[bench]   parity on {'all ' if rows is None else ''}{n_rows} rows: max |err| {err.max():.3e} ok={ok} "
        f"(oracle {t_oracle:.2f} s on {cpu_threads()} threads)")
    rec = {
        "workload": name, "path": plan["path"], "splits": plan["splits"], "kv_buffers": kv_buffers,
        "value": round(value, 3), "unit": unit, "ms_per_call": round(ms_call, 6), "calls": n,
        ("bytes_per_call" if bound == "hbm" else "flops_per_call"): work,
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(main_kernel, name) if main_kernel in KERNEL_SOURCES else None,
                     "kernel": main_kernel,
                     ("bytes_per_launch" if bound == "hbm" else "flops_per_launch"): work,
                     "avg_launch_us": round(kern_s * 1e6, 3),
                     "band_launch_us": round(b_ms / b_n * 1e3, 3) if b_n else None,
                     "combine_us": round(c_ms / c_n * 1e3, 3) if c_n else None},
        "parity": {"rows": n_rows, "all_rows": rows is None, "max_abs_err": float(err.max()), "ok": ok,
                   "oracle_s": round(t_oracle, 3), "oracle_threads": cpu_threads()},
    }
    del kv, qd, out, ws
    torch.cuda.empty_cache()
    return rec


def mla_work(w):
    """Algorithmic bytes and flops of one latent-attention call and of its
    split kernel alone. Visible latent rows are read once for all heads; the
    split kernel reads them and q_abs and writes (m, l, acc) per split (left
    out: workspace traffic is not algorithmic). Flops: absorbing q
    (2 H N R per row), scores and weighted sum (2 (R+P) + 2 R per visible
    (row, key, head)), and v_b (2 H Dv R per row)."""
    import numpy as np
    R, P, N, Dv, H, T = w.kv_rank, w.qk_rope, w.qk_nope, w.v_head_dim, w.heads, w.T
    pos = (w.posOffset or 0) + np.arange(T, dtype=np.int64)
    causal = True if w.causal is None else w.causal
    s = np.arange(w.S, dtype=np.int64)
    pairs = 0
    rows_seen = np.zeros(w.S, dtype=bool)
    for p in pos:
        vis = np.ones(w.S, dtype=bool)
        if w.window:
            vis = ((s > p - w.window) if causal else (np.abs(p - s) <= w.window)) | (s < (w.sinks or 0))
        if causal:
            vis &= s <= p
        pairs += int(vis.sum())
        rows_seen |= vis
    latent = int(rows_seen.sum()) * (R + P) * 4
    weights = H * N * R * 4 + H * Dv * R * 4
    io = T * H * (N + P) * 4 + T * H * Dv * 4
    split_flops = H * pairs * (2 * (R + P) + 2 * R)
    flops = split_flops + 2 * T * H * N * R + 2 * T * H * Dv * R
    return {"bytes": latent + weights + io, "flops": flops,
            "split_bytes": latent + T * H * (R + P) * 4, "split_flops": split_flops}


def run_mla(w, args, n_buffers):
    """Time attn_mla_forward on one latent workload: the three kernels' durations
    from dispatch-stamped events, the call time from a plain loop over
    rotated state copies; the split kernel rated against HBM or the fp32
    matrix peak, whichever bounds it; sampled heads checked against the oracle."""
    import numpy as np
    import torch

    import gqa_scaled_dot_amd as ga
    from oracle import mla as oracle_mla

    params = w.params()
    dev = torch.device("cuda:0")
    q, state, k_b, v_b = w.tensors()
    plan = ga.attn_mla_plan(w.T, w.S, **params)
    log(f"[bench] workload: {w.name}; plan {plan}")
    qd = torch.from_numpy(q).to(dev)
    sd = torch.from_numpy(state).to(dev)
    bufs = [(sd if i == 0 else sd.clone(), torch.from_numpy(k_b).to(dev), torch.from_numpy(v_b).to(dev))
            for i in range(n_buffers)]
    out = torch.empty((w.T, w.heads * w.v_head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ga.attn_mla_workspace_size(w.T, w.S, **params), 256), dtype=torch.uint8, device=dev)
    calls = [ga.prepare_mla_forward(qd, sb, kb, vb, out=out, workspace=ws, **params) for sb, kb, vb in bufs]
    n = args.steps
    for i in range(max(2, args.warmup // 5)):
        calls[i % n_buffers]()
    torch.cuda.synchronize()
    names = ("mla_absorb", "mla_split", "mla_combine")
    ga.attn_timing_enable(True)
    for name in names:
        ga.attn_timing_collect(name)
    for i in range(n):
        calls[i % n_buffers]()
    torch.cuda.synchronize()
    kern_us = {}
    for name in names:
        ms, cnt = ga.attn_timing_collect(name)
        kern_us[name] = round(ms / max(cnt, 1) * 1e3, 3)
    ga.attn_timing_enable(False)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        calls[i % n_buffers]()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / n
    work = mla_work(w)
    split_s = kern_us["mla_split"] * 1e-6
    # The split kernel's bound: its bytes at HBM peak against its flops at the matrix peak.
    t_hbm = work["split_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["split_flops"] / (FP32_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(work["split_bytes"] / split_s / 1e9, 3), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "bytes_per_launch": work["split_bytes"]}
    else:
        roof = {"bound": "mfma", "achieved": round(work["split_flops"] / split_s / 1e12, 3),
                "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "flops_per_launch": work["split_flops"]}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic("mla_split", w.name)
    roof["kernel"] = "mla_split"
    roof["avg_launch_us"] = kern_us["mla_split"]
    call_gbs = work["bytes"] / (ms_call * 1e-3) / 1e9
    call_tf = work["flops"] / (ms_call * 1e-3) / 1e12
    log(f"[bench]   call {ms_call * 1e3:.1f} us ({call_gbs:.0f} GB/s, {call_tf:.1f} TFLOP/s); kernels {kern_us}; "
        f"mla_split {roof['achieved']} {roof['unit']} = {roof['frac']:.1%} of {roof['peak']}")
    got = out.cpu().numpy().astype(np.float64)
    N, P, Dv = w.qk_nope, w.qk_rope, w.v_head_dim
    heads = sorted(set([0, w.heads - 1] + [int(x) for x in np.random.default_rng(5).integers(0, w.heads, 4)]))
    worst = 0.0
    ok = True
    for h in heads:
        qh = np.ascontiguousarray(q[:, h * (N + P):(h + 1) * (N + P)])
        ref = oracle_mla.mla_attention(qh, state, k_b[h:h + 1], v_b[h:h + 1], **w.replace(heads=1).params())
        err = np.abs(got[:, h * Dv:(h + 1) * Dv] - ref)
        worst = max(worst, float(err.max()))
        ok = ok and bool(np.all(err <= 1e-4 + 1e-4 * np.abs(ref)))
    log(f"[bench]   parity on heads {heads}: max |err| {worst:.3e} ok={ok}")
    rec = {"workload": w.name, "path": plan["path"], "splits": plan["splits"], "state_buffers": n_buffers,
           "value": round(call_gbs, 3), "unit": "GB/s", "ms_per_call": round(ms_call, 6), "calls": n,
           "bytes_per_call": work["bytes"], "flops_per_call": work["flops"], "tflops": round(call_tf, 3),
           "kernel_us": kern_us, "roofline": roof,
           "parity": {"heads": heads, "max_abs_err": worst, "ok": ok}}
    del bufs, qd, sd, out, ws
    torch.cuda.empty_cache()
    return rec


ROPE_Q_WORKLOAD = "llama3 rope on a prefill's q [4096, 4096]"
LLAMA3_ROPE = dict(base=500000.0, scaling=dict(rope_type="llama3", factor=8.0, low_freq_factor=1.0,
                                               high_freq_factor=4.0,
                                               original_max_position_embeddings=8192))


def run_rope(args):
    """The Llama-shaped decode step with the rotary embedding fused in (K rotated
    as it is written, q as attention loads it), and the standalone rope kernel
    on a prefill-sized q [4096, 32*128], rated against HBM."""
    import numpy as np
    import torch

    import gqa_scaled_dot_amd as ga
    import oracle
    import workloads

    w = workloads.LLAMA_DECODE
    params = w.params()
    dev = torch.device("cuda:0")
    q, k, v, _ = w.tensors()
    rp = dict(headDim=w.headDim, **LLAMA3_ROPE)
    n_buf = 2
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    kc = [torch.empty_like(kd) for _ in range(n_buf)]
    vc = [torch.empty_like(vd) for _ in range(n_buf)]
    for b in range(n_buf):
        ga.attn_rope_cache_write(kc[b], kd[:w.S - 1], 0, rp)
        ga.attn_cache_write(vc[b], vd[:w.S - 1], 0)
    new_k, new_v = kd[w.S - 1:], vd[w.S - 1:]
    out = torch.empty((w.T, w.heads * w.Dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ga.attn_workspace_size(w.T, w.S, **params), 256), dtype=torch.uint8, device=dev)
    # The step: the new K row turned at position S-1 into a one-row staging
    # buffer, then attn_forward_append (both rows written by the decode
    # kernel, q turned as it is loaded). Also timed: the same step as
    # attn_rope_cache_write (K) + cache_write (V) + attn_forward.
    k_rot = torch.empty_like(new_k)
    steps = [(ga.prepare_rope_cache_write(k_rot, new_k, 0, dict(rp, offset=w.S - 1)),
              ga.prepare_forward_append(qd, kc[b], vc[b], k_rot, new_v, w.S - 1, out=out, workspace=ws,
                                        q_rope=dict(LLAMA3_ROPE), **params)) for b in range(n_buf)]
    separate = [(ga.prepare_rope_cache_write(kc[b], new_k, w.S - 1, rp),
                 ga.prepare_cache_write(vc[b], new_v, w.S - 1),
                 ga.prepare_forward(qd, kc[b], vc[b], out=out, workspace=ws, q_rope=dict(LLAMA3_ROPE),
                                    **params)) for b in range(n_buf)]

    def step(i, calls=steps):
        for c in calls[i % n_buf]:
            c()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ga.attn_timing_enable(True)
    for name in ("decode_split", "combine", "rope", "cache_write"):
        ga.attn_timing_collect(name)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t = {name: ga.attn_timing_collect(name) for name in ("decode_split", "combine", "rope", "cache_write")}
    ga.attn_timing_enable(False)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    for i in range(args.warmup):
        step(i, separate)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i, separate)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_separate = e0.elapsed_time(e1) / args.steps
    for i in range(2):  # leave `out` as the step computes it
        step(i)
    torch.cuda.synchronize()
    us = {name: round(ms / max(n, 1) * 1e3, 3) for name, (ms, n) in t.items()}
    log(f"[bench] decode step with fused rope: {ms_step * 1e3:.2f} us (as three calls {ms_separate * 1e3:.2f} us); "
        f"kernels {us}")
    # The oracle on the same step: K rotated at positions 0..S-1, q at S-1.
    k_rot = oracle.rope(k, offset=0, **rp).astype(np.float32)
    q_rot = oracle.rope(q, offset=w.posOffset, **rp).astype(np.float32)
    ref = oracle.attention(q_rot, k_rot, v, threads=cpu_threads(), **params)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    ok = bool(np.all(err <= 1e-4 + 1e-4 * np.abs(ref)))
    log(f"[bench]   parity vs oracle: max |err| {err.max():.3e} ok={ok}")
    alg = decode_algorithmic_bytes(w)
    decode = {"workload": w.name + ", llama3 rope (theta 500000, factor 8) on q and the new K row",
              "step": "attn_rope_cache_write (new K row, into a staging row) + attn_forward_append(q_rope)",
              "ms_per_step": round(ms_step, 6), "value": round(alg / (ms_step * 1e-3) / 1e9, 1),
              "ms_per_step_separate_calls": round(ms_separate, 6),
              "separate_calls": "attn_rope_cache_write (new K row) + cache_write (new V row) + attn_forward(q_rope)",
              "unit": "GB/s", "kernel_us": us,
              "parity": {"max_abs_err": float(err.max()), "ok": ok}}
    del kc, vc, kd, vd, steps, separate, k_rot
    torch.cuda.empty_cache()

    # Standalone rope over a prefill's q: every element read and written once.
    wp = workloads.LLAMA_PREFILL
    x = workloads.normal((wp.T, wp.heads * wp.headDim), wp.seed, 0)
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    rq = dict(headDim=wp.headDim, **LLAMA3_ROPE)
    for _ in range(3):
        ga.attn_rope(xd, out=yd, **rq)
    torch.cuda.synchronize()
    ga.attn_timing_enable(True)
    ga.attn_timing_collect("rope")
    for _ in range(args.prefill_steps):
        ga.attn_rope(xd, out=yd, **rq)
    torch.cuda.synchronize()
    r_ms, r_n = ga.attn_timing_collect("rope")
    ga.attn_timing_enable(False)
    nbytes = 2 * x.size * 4
    kern_s = r_ms / r_n * 1e-3
    achieved = nbytes / kern_s / 1e9
    # Every row against the oracle (row t sits at position t).
    rows = sampled_rows(wp) if args.sampled_parity else list(range(wp.T))
    refr = oracle.rope(x, offset=0, **rq)[rows]
    errr = np.abs(yd.cpu().numpy()[rows].astype(np.float64) - refr)
    okr = bool(np.all(errr <= 4e-6 + 4e-6 * np.abs(refr)))
    log(f"[bench] rope kernel on q [{wp.T}, {wp.heads * wp.headDim}]: {kern_s * 1e6:.1f} us, "
        f"{achieved:.1f} GB/s = {achieved / HBM_PEAK_GBS:.1%} of 8 TB/s; parity max |err| {errr.max():.2e} ok={okr}")
    kernel = {"workload": ROPE_Q_WORKLOAD,
              "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("rope", ROPE_Q_WORKLOAD),
                           "kernel": "rope", "bytes_per_launch": nbytes,
                           "avg_launch_us": round(kern_s * 1e6, 3)},
              "parity": {"rows": len(rows), "max_abs_err": float(errr.max()), "ok": okr}}
    return {"decode_step": decode, "kernel": kernel}


# The relative-position bench lines: (workload, term kind, K/V copies, label).
RELPOS_LINES = {
    "LLAMA_DECODE_T5BIAS": ("LLAMA_DECODE", "position_bias", 2,
                            "llama3-8b-shaped decode with a T5-style bucketed position bias "
                            "(32 buckets, max distance 128)"),
    "LLAMA_DECODE_RELKV": ("LLAMA_DECODE", "relative_kv", 2,
                           "llama3-8b-shaped decode with relative key/value embeddings (max distance 128)"),
    "LLAMA_CHUNKED_RELKV": ("LLAMA_CHUNKED", "relative_kv", 1,
                            "llama3-8b-shaped chunked prefill T=512 at 3584, S=4096, with relative key/value "
                            "embeddings (max distance 128)"),
}


def run_relpos(name, args):
    import workloads
    wname, kind, kv_buffers, label = RELPOS_LINES[name]
    w = getattr(workloads, wname)
    return run_config(w, args, kv_buffers=kv_buffers, extra=relpos_terms(w, kind), label=label)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle timing")
    ap.add_argument("--no-configs", action="store_true",
                    help="only the Llama-shaped decode and prefill, not the other workloads")
    ap.add_argument("--sampled-parity", action="store_true",
                    help="check ~30 sampled rows of prefill-shaped outputs instead of every row")
    ap.add_argument("--only", default=None,
                    help="comma-separated workload names from workloads.py (e.g. LLAMA_CHUNKED,MLA_DECODE), "
                         "ROPE, or a relative-position line (LLAMA_DECODE_T5BIAS, LLAMA_DECODE_RELKV, "
                         "LLAMA_CHUNKED_RELKV): time just those, one record each, for profiling one kernel "
                         "and shape at a time")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op has no multi-GPU path in this library)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.prefill_steps < 1:
        ap.error("--steps and --prefill-steps must be >= 1 and --warmup >= 0")
    import workloads
    if args.only:
        names = [n.strip() for n in args.only.split(",")]
        for name in names:
            if name != "ROPE" and name not in RELPOS_LINES and getattr(workloads, name, None) is None:
                ap.error(f"--only: no workload named {name!r} in workloads.py (or ROPE, "
                         f"or one of {', '.join(RELPOS_LINES)})")
        calibration_copy()
        recs = []
        for name in names:
            if name == "ROPE":
                recs.append(run_rope(args))
                continue
            if name in RELPOS_LINES:
                recs.append(run_relpos(name, args))
                continue
            w = getattr(workloads, name)
            if isinstance(w, workloads.MlaWorkload):
                recs.append(run_mla(w, args, n_buffers=min(16, max(2, -(-(512 << 20) // mla_work(w)["bytes"])))))
            else:
                recs.append(run_config(w, args, kv_buffers=4 if w.T == 1 else 1))
        print(json.dumps({"metric": METRIC, "only": args.only, "configs": recs}), flush=True)
        return
    prefill = run_config(workloads.LLAMA_PREFILL, args)
    rec = run_decode(args)
    rec["prefill"] = prefill
    rec["rope"] = run_rope(args)
    if not args.no_configs:
        # The other workloads, each on its own plan (decode-shaped ones over 4
        # rotated K/V copies, as the Llama decode uses 2).
        rec["configs"] = [run_config(w, args, kv_buffers=4 if w.T == 1 else 1)
                          for w in (workloads.LLAMA_CHUNKED, workloads.GEMMA2_SWA,
                                    workloads.LATENT_DECODE, workloads.LATENT_NONCAUSAL,
                                    workloads.LLAMA_STREAMING, workloads.LLAMA70_DECODE,
                                    workloads.QWEN2_DECODE)]
        # Relative-position terms on the Llama-shaped decode and chunked prefill.
        rec["configs"] += [run_relpos(name, args) for name in RELPOS_LINES]
        # Latent attention in absorbed form; state copies rotate over >= 512 MiB of reads.
        rec["mla"] = [run_mla(w, args, n_buffers=min(16, max(2, -(-(512 << 20) // mla_work(w)["bytes"]))))
                      for w in (workloads.MLA_DECODE, workloads.MLA_DECODE_V3)]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
