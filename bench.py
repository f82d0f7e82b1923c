#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

One step = one attn_fwd call (the whole path: score product, masks, online
softmax, value product, log-sum-exp) over the s = 8192 workload
(B=1, H=32, d=128, causal, seeded bf16 inputs already resident in device
memory). Prints one JSON line:
  value          metric FLOPs (4*B*H*s^2*d, halved for causal) per second of
                 wall time over the timed steps, in TFLOP/s;
  roofline       the kernel's average launch duration from HIP events recorded
                 on the launch stream, against the bf16 dense MFMA peak;
                 its traffic is the HBM bytes per launch from rocprofv3
                 FETCH_SIZE / WRITE_SIZE passes, null once the kernel source
                 differs from the one they were taken on;
  cpu_baseline   the float64 CPU oracle, timed on a few heads of the same
                 workload on this host.

Before the W warm-up steps, --ramp-ms (default 100) of untimed back-to-back
steps bring the GPU to its sustained clock; the timed region is exactly K
steps. Options: --workload i selects another of the five workloads (for sweeps; the
default line is the s = 8192 one); --split-workload i --splits n times the
key-split entry point (attn_fwd_split: n key chunks, then their merge) on a
shape from workloads.SPLIT_WORKLOADS; a workload with key padding also reports
useful_tflops (FLOPs on the visible keys only); --calibrate-copy adds one plain device copy
of known size after the timed region, so a counter profile of this command also
holds the reference that scales FETCH_SIZE / WRITE_SIZE to bytes; --fp8
times the 8-bit-float forward (attn_fwd_fp8) on the same workload, its inputs
quantised per (batch item, head) to OCP E4M3 codes with float32 descale
factors, against the dense FP8 MFMA peak; --unfused times the materialising
path (attn_fwd_unfused: score matrix written to device memory, softmax in
place, value product) on the workload, with the fused forward timed beside it
for the ratio, against the HBM bandwidth peak. The default line also carries
the kernel's roofline fraction on the s = 4096 and s = 32768 causal workloads
and on the padded d = 64 one (`other_workloads`; --no-other-workloads skips
them, as the profiler commands do).
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s at 1 MI355X (s=4096–32768) + % of bf16 MFMA peak"
# MI355X dense bf16 MFMA: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
# MI355X dense FP8 MFMA: twice the bf16 rate
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS
# MI355X HBM3E bandwidth
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30
KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_44_amd", "csrc", "attn_fwd.hip")
KERNEL_SOURCE_FP8 = os.path.join(ROOT, "exact_attention_44_amd", "csrc", "attn_fwd_fp8.hip")

# HBM bytes per launch from two rocprofv3 counter passes (FETCH_SIZE, then
# WRITE_SIZE) of this script, each scaled by what the same counter reports for
# a 1 GiB copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); the mean over the
# launches after the first (the first runs with cold caches, the timed
# launches run back to back). Valid only for the kernel code they were taken
# on: reported as null once the code's hash (code_sha256: the source without
# its // comments and blank lines) differs.
def code_sha256(path: str) -> str:
    """sha256 of a C++/HIP source with its // comments, trailing blanks and
    blank lines removed: a comment-only edit keeps the hash."""
    lines = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


MEASURED_TRAFFIC = {
    "B=1,H=32,s=8192,d=128,causal": {
        "code_sha256": "c0082fdb6527b4d7105219e1931b1a969d364d0030029b3c5c8dadf104c03397",
        "fetch_bytes": 479501646,
        "write_bytes": 68157440,
        # SQ counter passes of the same command (mean over the launches after
        # the first; for the padded d=64 workload on an earlier source with
        # the same code for that kernel): MFMA-busy cycles per SIMD over SQ busy cycles per shader
        # engine (32 engines), the clock those busy cycles imply over the
        # launch, LDS bank conflicts, LDS instructions per wave and 64-key tile
        "counters": {
            "mfma_busy_frac": 0.688,
            "sustained_clock_ghz": 1.68,
            "lds_bank_conflicts": 0,
            "lds_instructions_per_wave_tile": 48,
        },
    },
    "B=4,H=16,s=2048,d=64,key-padding": {
        "code_sha256": "c0082fdb6527b4d7105219e1931b1a969d364d0030029b3c5c8dadf104c03397",
        "fetch_bytes": 64767271,
        "write_bytes": 17301504,
        "counters": {
            "mfma_busy_frac": 0.338,
            "sustained_clock_ghz": 2.17,
            "lds_bank_conflicts": 0,
            "lds_instructions_per_wave_tile": 19.5,
        },
    },
    "B=1,H=32,s=4096,d=128,causal": {
        "code_sha256": "c0082fdb6527b4d7105219e1931b1a969d364d0030029b3c5c8dadf104c03397",
        "fetch_bytes": 146159164,
        "write_bytes": 34079168,
    },
    "B=1,H=32,s=32768,d=128,causal,Kx3": {
        "code_sha256": "c0082fdb6527b4d7105219e1931b1a969d364d0030029b3c5c8dadf104c03397",
        "fetch_bytes": 4845509934,
        "write_bytes": 272638336,
    },
    "fp8:B=1,H=32,s=8192,d=128,causal": {
        "code_sha256": "e779acb56cc1bc5bf12e27322a1c62441d01eb6b48f0408f96a497cbe5aadf82",
        "fetch_bytes": 202676833,
        "write_bytes": 68177931,
    },
}


def algorithmic_bytes_of(w, mode: str) -> int:
    """HBM bytes one call must move at least: every input read once and every
    output written once (for the materialising path, also its score matrix:
    written, read and rewritten in place, read again, 2 bytes per score each
    time)."""
    B, H, s_q, s_k, d = w.B, w.H, w.s_q, w.s_k, w.d
    out_lse = 2 * B * H * s_q * d + 4 * B * H * s_q
    if mode == "unfused":
        return 8 * B * H * s_q * s_k + 2 * B * H * (s_q + 2 * s_k) * d + out_lse
    if mode == "fp8":  # E4M3 q, k, v (one byte each) and three float32 descales per head
        return B * H * (s_q + 2 * s_k) * d + 12 * B * H + out_lse
    if mode == "backward":  # read q, out, dout, k, v, lse; write dq, dk, dv
        return 2 * B * H * (3 * s_q + 2 * s_k) * d + 4 * B * H * s_q + 2 * B * H * (s_q + 2 * s_k) * d
    if mode == "forward":
        return 2 * B * H * (s_q + 2 * s_k) * d + out_lse
    raise ValueError(mode)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-ms", type=float, default=100.0,
                    help="untimed back-to-back steps before the warm-up steps, so the "
                         "GPU reaches its sustained clock (it needs ~25 ms of load)")
    ap.add_argument("--workload", type=int, default=2, help="index into workloads.WORKLOADS")
    ap.add_argument("--split-workload", type=int, default=None,
                    help="index into workloads.SPLIT_WORKLOADS: time the key-split entry point "
                         "(attn_fwd_split) on that shape instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (attn_bwd) of the workload instead; FLOPs "
                         "counted as 2.5x the forward's (five products of its size, one of "
                         "them the recomputed scores)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the 8-bit-float forward (attn_fwd_fp8) on E4M3-quantised "
                         "inputs of the workload instead")
    ap.add_argument("--unfused", action="store_true",
                    help="time the materialising forward (attn_fwd_unfused) on the workload "
                         "instead, and the fused forward beside it for the ratio")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the short timings of the other forward workloads")
    ap.add_argument("--splits", type=int, default=4,
                    help="key chunks for --split-workload (1 = the plain launch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true")
    return ap.parse_args()


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def time_launches(step, stream, n, ramp_ms=50.0):
    """Average and minimum duration (ms) of n launches of `step`, each between
    two HIP events on `stream`, after ramp_ms of untimed launches."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ramp_ms:
        step()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    return sum(ms) / len(ms), min(ms)


def other_workloads(E, dev, stream, skip_name):
    """Kernel roofline fractions of attn_fwd on the other forward workloads of
    the metric's range (s = 4096 and s = 32768 causal) and on the padded
    d = 64 one: seeded inputs, 30 launches each timed with HIP events."""
    import numpy as np
    import torch

    from workloads import WORKLOADS, generate
    res = {}
    for w in WORKLOADS[1:]:
        if w.name == skip_name:
            continue
        g = generate(w)
        q, k, v = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
        del g["q"], g["k"], g["v"]
        kpm = None if g["kpm"] is None else torch.from_numpy(g["kpm"]).to(dev)
        out = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.s_q), dtype=torch.float32, device=dev)
        args = (q, k, v, out, lse, w.B, w.H, w.s_q, w.s_k, w.d, float(g["scale"]), w.causal, kpm,
                stream.cuda_stream)

        def step():
            st = E.attn_fwd(*args)
            if st != E.ATTN_OK:
                raise E.AttnError(st)
        avg, mn = time_launches(step, stream, 30)
        r = {"kernel_avg_ms": round(avg, 5), "kernel_min_ms": round(mn, 5),
             "achieved_tflops": round(w.flops() / (avg * 1e-3) / 1e12, 2),
             "frac": round(w.flops() / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        if w.padded:
            useful = sum(4.0 * w.H * w.s_q * int(n) * w.d for n in g["lengths"])
            r["useful_frac"] = round(useful / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        res[w.name] = r
        del q, k, v, out, lse, kpm
        torch.cuda.empty_cache()
    return res


def cpu_baseline(w, g, target_s, backward=False, fp8=None):
    """Time the oracle on whole heads of the same workload until ~target_s
    (its gradients, with a seeded output gradient, for the backward pass; the
    E4M3 oracle on the quantised inputs `fp8` for the 8-bit-float forward)."""
    import numpy as np

    from oracle import attention_backward_fp64, attention_fp64, attention_fp8_fp64
    from workloads import bf16_bits_to_f32

    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = blas[0]
    except Exception:
        pass
    per_head = w.flops() / (w.B * w.H) * (2.5 if backward else 1.0)
    heads, spent = 0, 0.0
    rng = np.random.default_rng(w.seed + 2)
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = (bf16_bits_to_f32(g[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v"))
            kpm = None if g["kpm"] is None else g["kpm"][b:b + 1]
            if fp8 is not None:
                sl = (slice(b, b + 1), slice(h, h + 1))
                t0 = time.perf_counter()
                attention_fp8_fp64(*(fp8[n + "8"][sl] for n in ("q", "k", "v")),
                                   *(fp8["d" + n][sl] for n in ("q", "k", "v")),
                                   float(g["scale"]), w.causal, kpm)
            elif backward:
                dout = rng.standard_normal(q.shape)
                t0 = time.perf_counter()
                attention_backward_fp64(q, k, v, dout, float(g["scale"]), w.causal, kpm)
            else:
                t0 = time.perf_counter()
                attention_fp64(q, k, v, float(g["scale"]), w.causal, kpm)
            spent += time.perf_counter() - t0
            heads += 1
            if spent >= target_s:
                break
        if spent >= target_s:
            break
    return {
        "value": round(per_head * heads / spent / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "openblas_num_threads": os.environ.get("OPENBLAS_NUM_THREADS"),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle{' gradients' if backward else ''}"
                   f"{' on E4M3 inputs' if fp8 is not None else ''} (materialises each head's s x s scores, row blocks "
                   f"of 2048) on {heads} of {w.B * w.H} heads of {w.name}: {spent:.1f} s on "
                   f"{threads} BLAS threads of {os.cpu_count()} host CPUs ({cpu_model()}); "
                   f"FLOPs counted with the metric formula"),
    }


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "the kernel shards over (batch, head) with no communication, so N GPUs run "
              "the same single-GPU launch on their own heads.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_44_amd as E
    from workloads import SPLIT_WORKLOADS, WORKLOADS

    E.load_library()
    split = a.split_workload is not None
    w = SPLIT_WORKLOADS[a.split_workload] if split else WORKLOADS[a.workload]
    from workloads import generate
    g = generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (torch.from_numpy(g[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
    kpm = None if g["kpm"] is None else torch.from_numpy(g["kpm"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.s_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    args = (q, k, v, out, lse, w.B, w.H, w.s_q, w.s_k, w.d, float(g["scale"]), w.causal, kpm,
            stream.cuda_stream)

    fp8 = None
    if a.fp8:
        from workloads import bf16_bits_to_f32, quantize_heads_e4m3
        fp8 = {}
        for n in ("q", "k", "v"):
            fp8[n + "8"], fp8["d" + n] = quantize_heads_e4m3(bf16_bits_to_f32(g[n]))
        q8, k8, v8 = (torch.from_numpy(fp8[n + "8"]).to(dev) for n in ("q", "k", "v"))
        dq8, dk8, dv8 = (torch.from_numpy(fp8["d" + n]).to(dev) for n in ("q", "k", "v"))

        def step():
            st = E.attn_fwd_fp8(q8, k8, v8, dq8, dk8, dv8, out, lse, w.B, w.H, w.s_q, w.s_k, w.d,
                                float(g["scale"]), w.causal, kpm, stream.cuda_stream)
            if st != E.ATTN_OK:
                raise E.AttnError(st)
    elif a.backward:
        # forward outputs and a seeded output gradient, before any timing
        st = E.attn_fwd(*args)
        if st != E.ATTN_OK:
            raise E.AttnError(st)
        from workloads import round_to_bf16
        gnp = round_to_bf16(np.random.default_rng(w.seed + 1).standard_normal(
            (w.B, w.H, w.s_q, w.d), dtype=np.float32))
        dout = torch.from_numpy(gnp.view(np.int16)).view(torch.bfloat16).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws_bytes = E.attn_bwd_workspace_bytes(w.B, w.H, w.s_q)
        bws = torch.empty(max(bws_bytes, 256), dtype=torch.uint8, device=dev)

        def step():
            st = E.attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, w.B, w.H, w.s_q, w.s_k, w.d,
                            float(g["scale"]), w.causal, kpm, bws, bws.numel(), stream.cuda_stream)
            if st != E.ATTN_OK:
                raise E.AttnError(st)
    elif a.unfused:
        s_bytes = E.attn_fwd_unfused_workspace_bytes(w.B, w.H, w.s_q, w.s_k)
        scores = torch.empty(max(s_bytes, 16), dtype=torch.uint8, device=dev)  # outside the timed region

        def step():
            st = E.attn_fwd_unfused(*args[:13], scores, s_bytes, args[13])
            if st != E.ATTN_OK:
                raise E.AttnError(st)
    elif split:
        chunks = max(1, min(a.splits, (w.s_k + 63) // 64))
        ws_bytes = E.attn_fwd_split_workspace_bytes(w.B, w.H, w.s_q, w.d, chunks)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # outside the timed region

        def step():
            st = E.attn_fwd_split(*args[:13], a.splits, ws, ws_bytes, args[13])
            if st != E.ATTN_OK:
                raise E.AttnError(st)
    else:
        def step():
            st = E.attn_fwd(*args)
            if st != E.ATTN_OK:
                raise E.AttnError(st)

    t_ramp = time.perf_counter()
    ramp_steps = 0
    while (time.perf_counter() - t_ramp) * 1e3 < a.ramp_ms:
        for _ in range(5):
            step()
        ramp_steps += 5
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)

    if a.calibrate_copy:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    fused_ms = None
    if a.unfused:
        def fused_step():
            st = E.attn_fwd(*args)
            if st != E.ATTN_OK:
                raise E.AttnError(st)
        fused_ms = time_launches(fused_step, stream, a.steps)[0]

    flops = w.flops() * (2.5 if a.backward else 1.0)
    mode = "unfused" if a.unfused else "fp8" if a.fp8 else "backward" if a.backward else "forward"
    algorithmic_bytes = algorithmic_bytes_of(w, mode)
    traffic, traffic_detail = None, {"algorithmic_bytes": algorithmic_bytes}
    measured = None if (a.backward or split or a.unfused) else \
        MEASURED_TRAFFIC.get(("fp8:" if a.fp8 else "") + w.name)
    if measured is not None:
        current = code_sha256(KERNEL_SOURCE_FP8 if a.fp8 else KERNEL_SOURCE)
        if current == measured["code_sha256"]:
            traffic = measured["fetch_bytes"] + measured["write_bytes"]
            traffic_detail.update(fetch_bytes=measured["fetch_bytes"],
                                  write_bytes=measured["write_bytes"],
                                  code_sha256=current)
            if "counters" in measured:
                traffic_detail["counters"] = measured["counters"]
    value = flops * a.steps / wall / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if a.fp8 else PEAK_BF16_TFLOPS
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ramp_steps": ramp_steps,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "s_q": w.s_q, "s_k": w.s_k, "d": w.d,
                   "causal": w.causal, "key_padding": w.padded, "seed": w.seed,
                   "flops_per_step": flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch",
            "traffic_detail": traffic_detail,
            "kernel": ("attn_fwd_fp8_kernel" if a.fp8
                       else ("attn_bwd_dq_kernel + " + ("attn_bwd_dkv_pair_kernel" if w.d == 128
                                                         else "attn_bwd_dkv_kernel")) if a.backward
                       else "attn_fwd_kernel (key-split) + attn_merge_kernel" if split
                       else "attn_fwd_kernel"),
            "kernel_avg_ms": round(kern_avg_ms, 5),
            "kernel_min_ms": round(min(kern_ms), 5),
        },
    }
    if a.fp8:
        res["config"]["entry_point"] = "attn_fwd_fp8"
        res["config"]["inputs"] = "OCP E4M3 codes, per-(b, h) float32 descale"
        res["metric"] = METRIC.replace("% of bf16 MFMA peak", "% of FP8 MFMA peak") + " (FP8 forward)"
        res["dtype"] = "fp8-e4m3 products, fp32 accumulate, bf16 out"
        res["pct_of_fp8_peak"] = round(100.0 * value / PEAK_FP8_TFLOPS, 2)
        del res["pct_of_bf16_peak"]
    if a.unfused:
        gbs = algorithmic_bytes / (kern_avg_ms * 1e-3) / 1e9
        res["metric"] = METRIC.replace(" + % of bf16 MFMA peak", "") + " (unfused materialising path)"
        res["config"]["entry_point"] = "attn_fwd_unfused"
        res["roofline"].update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                               frac=round(gbs / PEAK_HBM_GBS, 4),
                               kernel="unf_scores_kernel + unf_softmax_kernel + unf_values_kernel "
                                      "(the three kernels of one call, timed together)")
        res["unfused"] = {
            "score_matrix_bytes": s_bytes,
            "score_matrix_gb": round(s_bytes / 1e9, 2),
            "fused_kernel_avg_ms": round(fused_ms, 5),
            "unfused_over_fused_time": round(kern_avg_ms / fused_ms, 3),
        }
        del res["pct_of_bf16_peak"]
    if a.backward:
        res["config"]["pass"] = "backward"
        res["metric"] = METRIC + " (backward pass: dq, dk, dv)"
    if split:
        res["config"]["n_splits"] = a.splits
        res["config"]["entry_point"] = "attn_fwd_split"
    if w.padded:
        # the metric's nominal FLOPs ignore padding; the work on visible keys only
        lengths = g["lengths"]
        useful = sum(4.0 * w.H * w.s_q * int(n) * w.d for n in lengths) * (2.5 if a.backward else 1.0)
        res["useful_tflops"] = round(useful * a.steps / wall / 1e12, 2)
    plain = not (a.fp8 or a.backward or split or a.unfused)
    if plain and not a.no_other_workloads:
        res["other_workloads"] = other_workloads(E, dev, stream, w.name)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, g, a.cpu_seconds, backward=a.backward, fp8=fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
