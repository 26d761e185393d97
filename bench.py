"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--all] [--copy-calibration]
    python bench.py --backward [--workload long_fwd_bwd] [--dtype bf16|f16] [--steps K]
                    [--warmup W]
    python bench.py --decode [--steps K] [--warmup W]
    python bench.py --fp8 [--steps K] [--warmup W]

One step = one fa_fwd call over the whole workload: work partition, Q/K/V
tile loads, QK^T, masking, online softmax, PV and the epilogue all run in the
one forward kernel.  The default workload is the GQA causal prefill (B=1,
Hq=32, Hkv=8, N=8192, d=128, bf16).  Inputs are seeded synthetic N(0,1) values
already resident in HBM when the timed region starts.  Timing uses HIP events
recorded on the stream the kernel runs on (torch's current stream).

Prints one JSON line with the throughput in attention TFLOP/s (4 B Hq Nq Nk d,
halved for causal), the roofline position of the forward kernel, and the CPU
oracle timed on this host on a bounded sample of the same workload.
With --backward it times only the backward call (D, dK/dV and dQ kernels) of
a workload that has one and prints one line with its time and throughput on
the five counted products (2.5x the forward count); this is the mode the
backward's kernel traces and counters are taken from.  --decode does the
same for the split-KV decode workload (split and combine kernels), --fp8 for
the FP8 forward of the GQA prefill shape and the quantizer that makes its
inputs.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: twice the bf16 rate
METRIC = "attention TFLOP/s + % of bf16 MFMA peak, causal fwd N=8192 d=128 GQA"
# the forward kernel's sources and the build script that sets its code-generation
# options (paths relative to the package's csrc/)
FWD_SOURCES = ["fa_fwd_kernel.h", "fa_fwd_bf16.hip", "fa_fwd_bf16_d128.hip", "fa_device.h",
               "fa_params.h", "../build.py"]


def attention_flops(inp):
    """Algorithmic forward FLOPs: 4 B Hq Nq Nk d, halved for causal; for
    windowed packed batches 4 Hq d times the exact number of visible pairs."""
    d, hq = inp["d"], inp["Hq"]
    if inp.get("cu_seqlens") is None and inp.get("window", 0) <= 0:
        f = 4.0 * inp["B"] * hq * inp["Nq"] * inp["Nk"] * d
        return f / 2 if inp["causal"] else f
    lengths = (np.diff(inp["cu_seqlens"]) if inp.get("cu_seqlens") is not None
               else [inp["Nq"]] * inp["B"])
    W = inp.get("window", 0)
    pairs = 0
    for L in lengths:
        L = int(L)
        if inp["causal"]:
            pairs += L * (L + 1) // 2 if (W <= 0 or L <= W) else W * (W + 1) // 2 + (L - W) * W
        else:
            pairs += L * L if W <= 0 else sum(L - max(0, i - W + 1) for i in range(L))
    return 4.0 * hq * d * pairs


def algorithmic_bytes(inp):
    """Bytes the forward must move: Q, K, V read once, O and LSE written once."""
    e = 4 if inp["dtype"] == "f32" else 2
    nq = inp["q"].size
    nk = inp["k"].size
    rows = inp["q"].shape[0] * (inp["q"].shape[1] if inp["q"].ndim == 4 else 1)
    bias = 0 if inp.get("bias") is None else inp["bias"].nbytes  # read once at least
    return e * (2 * nq + 2 * nk) + 4 * rows * inp["Hq"] + bias


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_28_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current forward-kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_bf16_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(FWD_SOURCES):
        return None
    return float(m_bytes.group(1))


def blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        n = [x["num_threads"] for x in info if x.get("user_api") == "blas"]
        return int(n[0]) if n else 1
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(inp, budget_s=12.0):
    """The fp64 oracle on whole heads of the same workload, until the budget
    is spent; rate in the same algorithmic FLOP units as the GPU figure."""
    import oracle
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, N, hq, d = q.shape
    hkv = k.shape[2]
    per_head = attention_flops(dict(inp, B=1, Hq=1))
    t0 = time.perf_counter()
    done = 0
    for b in range(B):
        for h in range(hq):
            g = oracle.kv_head_of(h, hq, hkv)
            oracle.attn_fwd_rows(q[b, :, h], k[b, :, g], v[b, :, g], np.arange(N),
                                 inp["scale"], inp["causal"], inp["window"])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    return {"value": per_head * done / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{done} of {B * hq} (batch, query head) pairs, all {N} rows each, "
                      f"fp64 NumPy, {dt:.1f} s"}


def device_inputs(inp):
    import torch
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[inp["dtype"]]
    mk = lambda x: torch.from_numpy(x).to(dt).cuda()
    out = {n: mk(inp[n]) for n in ("q", "k", "v")}
    cu = inp.get("cu_seqlens")
    out["cu"] = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    out["bias"] = None if inp.get("bias") is None else torch.from_numpy(inp["bias"]).cuda()
    return out


# The GPU clock ramps up over the first ~100 ms of sustained work: a few
# warm-up launches leave the timed region partly at a low clock.  Warm-up
# therefore runs at least --warmup launches and at least this long.
MIN_WARMUP_MS = 300.0


def warm_up(launch, warmup, min_ms=MIN_WARMUP_MS):
    """Run `warmup` launches, then more in batches of 10 until `min_ms` of
    wall time has passed; returns the number of launches."""
    import torch
    t0 = time.perf_counter()
    n = 0
    for _ in range(warmup):
        launch()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            launch()
            n += 1
        torch.cuda.synchronize()
    return n


def timed(launch, steps, stream):
    """Time exactly `steps` launches with HIP events on `stream`: one event
    before the first and one after each launch.  Returns (ms per launch over
    the whole region, per-launch ms)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        launch()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def time_forward(inp, dev, steps, warmup, stats=None):
    import torch
    import exact_io_aware_28_amd as fa
    fn = {"bf16": fa.fa_fwd, "f16": fa.fa_fwd_f16, "f32": fa.fa_fwd_f32}[inp["dtype"]]
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"],
              cu_seqlens=dev["cu"], max_seqlen=inp["Nq"] if dev["cu"] is not None else None)
    if dev.get("bias") is not None:  # same call with the bias in place of cu_seqlens
        bias = dev["bias"]
        kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"])
        fn = lambda q, k, v, **a: fa.fa_fwd_bias(q, k, v, bias, **a)
    if inp.get("dropout_p"):
        dp, ds = inp["dropout_p"], inp["dropout_seed"]
        fn = lambda q, k, v, **a: fa.fa_fwd_dropout(q, k, v, dp, ds, **a)
    o, lse = fn(dev["q"], dev["k"], dev["v"], **kw)
    launch = lambda: fn(dev["q"], dev["k"], dev["v"], out=o, lse=lse, **kw)
    n_warm = warm_up(launch, warmup)
    ms, per = timed(launch, steps, torch.cuda.current_stream())
    if stats is not None:
        srt = sorted(per)
        stats.update(warmup_launches=n_warm,
                     launch_ms={"first": round(per[0], 5), "last": round(per[-1], 5),
                                "min": round(srt[0], 5), "median": round(srt[len(srt) // 2], 5),
                                "max": round(srt[-1], 5)})
    return ms  # ms per step (= per launch)


def time_backward(inp, dev, steps, warmup):
    import torch
    import exact_io_aware_28_amd as fa
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"],
              cu_seqlens=dev["cu"], max_seqlen=inp["Nq"] if dev["cu"] is not None else None)
    fwd, bwd = {"bf16": (fa.fa_fwd, fa.fa_bwd), "f16": (fa.fa_fwd_f16, fa.fa_bwd_f16)}[
        inp["dtype"]]
    if dev.get("bias") is not None:
        bias = dev["bias"]
        kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"])
        fwd = lambda q, k, v, **a: fa.fa_fwd_bias(q, k, v, bias, **a)
        bwd = lambda q, k, v, o, do, lse, **a: fa.fa_bwd_bias(q, k, v, bias, o, do, lse, **a)
    if inp.get("dropout_p"):
        dp, ds = inp["dropout_p"], inp["dropout_seed"]
        fwd = lambda q, k, v, **a: fa.fa_fwd_dropout(q, k, v, dp, ds, **a)
        bwd = lambda q, k, v, o, do, lse, **a: fa.fa_bwd_dropout(q, k, v, o, do, lse, dp, ds,
                                                                 **a)
    o, lse = fwd(dev["q"], dev["k"], dev["v"], **kw)
    do = torch.from_numpy(inp["do"]).to(dev["q"].dtype).cuda()
    dq, dk, dv = bwd(dev["q"], dev["k"], dev["v"], o, do, lse, **kw)
    ws = torch.empty(fa.fa_bwd_workspace_size(inp["B"] * inp["Nq"], inp["Hq"], inp["d"]),
                     dtype=torch.uint8, device="cuda")
    launch = lambda: bwd(dev["q"], dev["k"], dev["v"], o, do, lse, dq=dq, dk=dk, dv=dv,
                         workspace=ws, **kw)
    warm_up(launch, warmup)
    return timed(launch, steps, torch.cuda.current_stream())[0]


def decode_pairs(inp):
    """Visible (query row, key) pairs per head of a decode workload, summed
    over sequences (bottom-right causal: row i sees i + L - Nq + 1 keys)."""
    nq = inp["Nq"]
    total = 0
    for L in np.asarray(inp["seqlens_k"], dtype=np.int64):
        for i in range(nq):
            seen = L if not inp["causal"] else min(L, max(0, i + L - nq + 1))
            if inp.get("window"):
                seen = min(seen, inp["window"])
            total += seen
    return total


def decode_bytes(inp):
    """Algorithmic bytes of one decode call: the K/V rows in use read once,
    Q read, O and LSE written (the split partials are not counted)."""
    B, hq, hkv, nq, d = (inp[x] for x in ("B", "Hq", "Hkv", "Nq", "d"))
    kv = int(np.asarray(inp["seqlens_k"], dtype=np.int64).sum()) * hkv * d * 2 * 2
    return kv + 2 * B * nq * hq * d * 2 + B * hq * nq * 4


def time_decode(inp, steps, warmup):
    import torch
    import exact_io_aware_28_amd as fa
    q = torch.from_numpy(inp["q"]).to(torch.bfloat16).cuda()
    k = torch.from_numpy(inp["k"]).to(torch.bfloat16).cuda()
    v = torch.from_numpy(inp["v"]).to(torch.bfloat16).cuda()
    lens = torch.from_numpy(np.asarray(inp["seqlens_k"], np.int32)).cuda()
    B, nq, hq, d = q.shape
    splits = fa.fa_decode_num_splits(B, hq, k.shape[2], nq, k.shape[1])
    ws = torch.empty(fa.fa_decode_workspace_size(B, hq, nq, d, splits), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device="cuda")
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"], seqlens_k=lens,
              num_splits=splits, out=o, lse=lse, workspace=ws)
    launch = lambda: fa.fa_decode(q, k, v, **kw)
    warm_up(launch, warmup + 1)
    return timed(launch, steps, torch.cuda.current_stream())[0], splits


def decode_line(name, steps, warmup):
    di = workloads.make_decode_inputs(name)
    dms, splits = time_decode(di, steps, warmup)
    gbs = decode_bytes(di) / (dms * 1e-3) / 1e9
    tf = 4.0 * di["Hq"] * di["d"] * decode_pairs(di) / (dms * 1e-3) / 1e12
    return {"workload": name, "direction": "decode", "ms": round(dms, 4), "GB/s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "TFLOP/s": round(tf, 2),
            "num_splits": splits, "algorithmic_bytes": decode_bytes(di)}


def time_fp8(name, steps, warmup):
    """FP8 forward over resident E4M3 codes and block scales, and the
    quantizer that makes them from bf16 (Q and K rotated, V transposed)."""
    import torch
    import exact_io_aware_28_amd as fa
    inp = workloads.make_fp8_inputs(name)
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().view(torch.float8_e4m3fn)
    q8, k8 = dev8(inp["q8"]), dev8(inp["k8"])
    vt8 = dev8(workloads.transpose_v8(inp["v8"]))
    sq, sk, sv = (torch.from_numpy(inp[n]).cuda() for n in ("sq", "sk", "sv"))
    o, lse = fa.fa_fwd_fp8(q8, k8, vt8, sq, sk, sv, causal=inp["causal"], window=inp["window"])
    launch = lambda: fa.fa_fwd_fp8(q8, k8, vt8, sq, sk, sv, causal=inp["causal"],
                                   window=inp["window"], out=o, lse=lse)
    warm_up(launch, warmup)
    ms = timed(launch, steps, torch.cuda.current_stream())[0]
    flops = attention_flops(dict(inp, cu_seqlens=None))
    # the quantizer over bf16 tensors of the same shapes
    B, N, hq, hkv, d = inp["B"], inp["Nq"], inp["Hq"], inp["Hkv"], inp["d"]
    xq = torch.randn(B, N, hq, d, device="cuda").to(torch.bfloat16)
    xk = torch.randn(B, N, hkv, d, device="cuda").to(torch.bfloat16)
    signs = (torch.randint(0, 2, (d,), device="cuda") * 2 - 1).float()
    qo, qs = fa.fa_quantize_fp8(xq, signs=signs)
    ko, ks = fa.fa_quantize_fp8(xk, signs=signs)
    vo, vs = fa.fa_quantize_fp8(xk, transpose=True)

    def quant():
        fa.fa_quantize_fp8(xq, signs=signs, out=qo, scales=qs)
        fa.fa_quantize_fp8(xk, signs=signs, out=ko, scales=ks)
        fa.fa_quantize_fp8(xk, transpose=True, out=vo, scales=vs)
    warm_up(quant, warmup)
    qms = timed(quant, steps, torch.cuda.current_stream())[0]
    # bytes moved: each bf16 element read (2 B) and its code written (1 B)
    qbytes = 3 * xq.numel() + 2 * 3 * xk.numel()
    return {"workload": name, "direction": "fwd", "dtype": "fp8-e4m3", "ms": round(ms, 4),
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_fp8_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "quantize_qkv_ms": round(qms, 4),
            "quantize_GB/s": round(qbytes / (qms * 1e-3) / 1e9, 1)}


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "reps": reps}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gqa_causal_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--all", action="store_true",
                    help="also time every other workload and the backward (extra lines)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time only the backward of --workload (default long_fwd_bwd)")
    ap.add_argument("--dtype", choices=["bf16", "f16"], default=None,
                    help="with --backward: operand type (default: the workload's, bf16)")
    ap.add_argument("--decode", action="store_true",
                    help="time only the split-KV decode workload")
    ap.add_argument("--fp8", action="store_true",
                    help="time only the FP8 forward of the GQA prefill shape and its "
                         "quantizer")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for --gpus {a.gpus}); "
              "the attention path shards over (sequence, KV-head) units with no "
              "communication, so a multi-GPU run is one independent run per GPU.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    import exact_io_aware_28_amd as fa
    fa.lib()  # fails loudly when the HIP library is missing

    if a.copy_calibration:
        copy_calibration()
        return 0

    if a.decode:
        for name in workloads.DECODE_WORKLOADS:
            print(json.dumps(decode_line(name, a.steps, a.warmup)), flush=True)
        return 0

    if a.fp8:
        print(json.dumps(time_fp8("gqa_causal_prefill_fp8", a.steps, a.warmup)), flush=True)
        return 0

    if a.backward:
        name = a.workload if a.workload != "gqa_causal_prefill" else "long_fwd_bwd"
        spec = dict(workloads.WORKLOADS[name])
        if a.dtype:
            spec["dtype"] = a.dtype
        wi = workloads.make_inputs(spec)
        if not wi.get("bwd"):
            print(f"bench.py: workload {name} has no backward", file=sys.stderr)
            return 2
        bms = time_backward(wi, device_inputs(wi), a.steps, a.warmup)
        tf = 2.5 * attention_flops(wi) / (bms * 1e-3) / 1e12
        print(json.dumps({"workload": name, "direction": "bwd", "dtype": wi["dtype"],
                          "steps": a.steps,
                          "warmup": a.warmup, "ms": round(bms, 4), "TFLOP/s": round(tf, 2),
                          "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)
        return 0

    inp = workloads.make_inputs(a.workload)
    dev = device_inputs(inp)
    stats = {}
    ms = time_forward(inp, dev, a.steps, a.warmup, stats)
    flops = attention_flops(inp)
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = traffic_from_profile(a.workload)
    cfg = {"workload": a.workload}
    for key in ("B", "Hq", "Hkv", "N", "d", "causal", "window", "nseq", "T"):
        if key in inp and key not in ("q", "k", "v"):
            cfg[key] = int(inp[key]) if not isinstance(inp[key], bool) else inp[key]
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp["dtype"],
        "data": "synthetic",
        "config": cfg,
        "warmup_launches": stats["warmup_launches"],
        "min_warmup_ms": MIN_WARMUP_MS,
        "launch_ms": stats["launch_ms"],
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbs_algorithmic": round(algorithmic_bytes(inp) / (ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "mfma",
            "kernel": "fwd_bf16_kernel",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": algorithmic_bytes(inp),
        },
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, a.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)

    if a.all:
        for name in workloads.WORKLOADS:
            if name == a.workload:
                continue
            wi = workloads.make_inputs(name)
            wd = device_inputs(wi)
            wms = time_forward(wi, wd, max(a.steps, 10), a.warmup)
            extra = {"workload": name, "direction": "fwd", "ms": round(wms, 4),
                     "TFLOP/s": round(attention_flops(wi) / (wms * 1e-3) / 1e12, 2),
                     "GB/s_algorithmic": round(algorithmic_bytes(wi) / (wms * 1e-3) / 1e9, 1)}
            print(json.dumps(extra), flush=True)
            if wi.get("bwd"):
                bms = time_backward(wi, wd, 5, 1)
                print(json.dumps({"workload": name, "direction": "bwd", "ms": round(bms, 4),
                                  "TFLOP/s": round(2.5 * attention_flops(wi) / (bms * 1e-3) / 1e12, 2)}),
                      flush=True)
            del wd
            torch.cuda.empty_cache()
        # the headline workload again with fp16 operands (same kernel body)
        wi = workloads.make_inputs(dict(workloads.WORKLOADS[a.workload], dtype="f16"))
        wd = device_inputs(wi)
        wms = time_forward(wi, wd, a.steps, a.warmup)
        print(json.dumps({"workload": a.workload, "direction": "fwd", "dtype": "f16",
                          "ms": round(wms, 4),
                          "TFLOP/s": round(attention_flops(wi) / (wms * 1e-3) / 1e12, 2)}),
              flush=True)
        del wd
        torch.cuda.empty_cache()
        # and the backward of the long workload with fp16 operands
        wi = workloads.make_inputs(dict(workloads.WORKLOADS["long_fwd_bwd"], dtype="f16"))
        wd = device_inputs(wi)
        bms = time_backward(wi, wd, 5, 1)
        print(json.dumps({"workload": "long_fwd_bwd", "direction": "bwd", "dtype": "f16",
                          "ms": round(bms, 4),
                          "TFLOP/s": round(2.5 * attention_flops(wi) / (bms * 1e-3) / 1e12, 2)}),
              flush=True)
        del wd
        torch.cuda.empty_cache()
        for name in workloads.FP8_WORKLOADS:
            print(json.dumps(time_fp8(name, max(a.steps, 10), a.warmup)), flush=True)
            torch.cuda.empty_cache()
        for name in workloads.DECODE_WORKLOADS:
            print(json.dumps(decode_line(name, max(a.steps, 10), a.warmup)), flush=True)
            torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
