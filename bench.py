#!/usr/bin/env python3
"""Benchmark of the hybrid W4A16 MoE layer (NVFP4/MXFP4 kept tier + NF3 tail) on
one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default run: both halves of the metric.
  * decode: the Qwen3-MoE-shaped layer (E=128, H=2048, I=768, top-8, 32 NVFP4 + 96
    NF3 experts) at M = 8 tokens per step -- `value` is its tokens/s -- with the
    M = 1, 2, 4 points of the decode sweep beside it;
  * prefill: the GLM-class layer (E=256, H=6144, I=2048, top-8, 64 NVFP4 + 192 NF3,
    skewed routing) at M = 4096, reported under "prefill" with its TFLOP/s.
  * W4A4: the GLM-class MXFP4 + NF3 layer at M = 512 with the kept tier's activations in
    MXFP4 on MX-scaled matrix cores, reported under "w4a4" beside the same layer as W4A16.
--workload NAME runs one workload alone: qwen_decode, glm_decode (M=8), glm_prefill
(M=4096), glm_mxfp4 (MXFP4 kept tier, M=512; --w4a4 for W4A4) or glm_uniform (no bit
map, M=512).

One step is one hybrid_moe_forward over one batch: routing, grouping or align,
both tiers' W13 + SwiGLU, W2 + weighted combine. Steps replay HIP graphs of the
forward that rotate over enough copies of the packed weights to exceed the
256 MB Infinity Cache, so every step reads its experts from HBM. Inputs are
synthetic (seeded), resident in HBM before timing starts.

Each workload carries a `roofline` of its dominant kernel (decode: the W13 GEMV;
prefill: the W13 grouped GEMM), bound by HBM or by the MFMA units as the layer's
arithmetic intensity says. Its `achieved`/`frac` use the kernel's average duration
from the committed rocprofv3 kernel trace (profiles/kernel_times.json) when that was
taken on the current kernel sources, and otherwise the live HIP-event timing of
back-to-back launches on the launch stream, which is always reported beside it.
`cpu_baseline` times the CPU oracle (median of 5 runs for decode, 3 for prefill) on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tok/s + HBM GB/s (M<=8); prefill TFLOP/s (M=4096)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 * 1024 * 1024
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload(name, m):
    import synth
    table = {"qwen_decode": synth.qwen_decode, "glm_decode": synth.glm_decode,
             "glm_prefill": synth.glm_prefill, "glm_mxfp4": synth.glm_mxfp4,
             "glm_uniform": synth.glm_uniform}
    fn = table[name]
    return fn() if m is None else fn(m)


def describe(w, packed):
    bm = packed["bit_map"]
    n_kept = w.E if bm is None else int((bm == 4).sum())
    kept = packed["kept_format"].upper()
    tiers = f"{n_kept} {kept} + {w.E - n_kept} NF3" if bm is not None else f"uniform {kept}"
    return f"{w.name}: E={w.E} H={w.H} I={w.I} top-{w.top_k} SwiGLU, {tiers}"


def expert_bytes(packed):
    """Packed bytes of one expert's W13 and W2 per tier: codes + scales + global."""
    out = {}
    for tier in ("kept", "nf3"):
        d = packed[tier]
        if d["w13_q"].shape[0] == 0:
            continue
        per = lambda key: d[key][0].nbytes if key in d else 0
        g = 4 if (tier == "kept" and packed["kept_format"] == "nvfp4") else 0
        out[tier] = {"w13": per("w13_q") + per("w13_s") + g, "w2": per("w2_q") + per("w2_s") + g}
    return out


def kernel_sources(decode, w4a4):
    """The source files of a workload's dominant kernel (what its profiles depend on)."""
    if decode:
        return ("decode.hip", "route_common.h", "device_common.h")
    if w4a4:
        return ("prefill.hip", "mx_gemm.h", "w4a4.hip", "device_common.h")
    return ("prefill.hip", "mx_gemm.h", "device_common.h")


def source_hash(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "weight_only_quantized_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_key, src_hash, launches_bytes):
    """HBM traffic per launch of the dominant kernel from committed rocprofv3 --pmc
    counts (profiles/pmc_traffic.json), or None if they were taken on other source."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        rec = data.get(kernel_key)
        if not rec or rec.get("source_hash") != src_hash:
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


def measure(w, steps, warmup, copies=None, stage_steps=30, packed=None, block_m=None,
            decode_launch=0, act_format=0):
    """Times `steps` graph replays of the forward at w.M; returns a result dict."""
    import numpy as np
    import torch

    import synth
    import weight_only_quantized_moe_amd as hm

    if packed is None:
        t0 = time.time()
        packed = synth.packed_layer(w)
        log(f"{w.name}: generated packed layer in {time.time() - t0:.1f}s")
    bm = packed["bit_map"]
    fmt = hm.KEPT_NVFP4 if packed["kept_format"] == "nvfp4" else hm.KEPT_MXFP4
    layer = hm.moe_layer_create(w.E, w.H, w.I, w.top_k, w.M, fmt, bm, block_m or 0, decode_launch,
                                act_format)
    block_m = hm.moe_layer_query(layer)["block_m"]
    base = hm.DeviceWeights(packed)
    layer_bytes = base.nbytes()
    if copies is None:
        copies = max(1, math.ceil(4 * MALL_BYTES / layer_bytes))
    wts = [base] + [base.clone() for _ in range(copies - 1)]
    scratch = torch.zeros(hm.moe_scratch_bytes(layer), dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(synth.activations_bf16(w, w.M).view(np.int16)).cuda()
    lg = torch.from_numpy(synth.router_logits(w, w.M)).cuda()
    y = torch.empty((w.M, w.H), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()

    # eager warm-up (also fills the decode view / align tables for the byte counts)
    for i in range(3):
        hm.hybrid_moe_forward(layer, wts[i % copies], x, lg, y, scratch)
    torch.cuda.synchronize()

    # one HIP graph per weight copy
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                hm.hybrid_moe_forward(layer, wts[c], x, lg, y, scratch)
            graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / steps

    # per-stage durations, live, with HIP events on the launch stream; a GPU sleep
    # first lets the host queue every launch so the kernels run back to back
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(stage_steps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for i in range(stage_steps):
        wt = wts[i % copies]
        ev[i][0].record()
        for st in range(4):
            hm.hybrid_moe_forward_stage(layer, wt, x, lg, y, scratch, st)
            ev[i][st + 1].record()
    torch.cuda.synchronize()
    stage_us = [sum(ev[i][st].elapsed_time(ev[i][st + 1]) for i in range(stage_steps)) * 1e3 / stage_steps
                for st in range(4)]

    # the dominant stage (W13) alone: back-to-back launches over the weight copies
    # between two events on the launch stream; the average is one launch's duration
    reps = max(30, stage_steps)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(1e8))
    k0.record()
    for i in range(reps):
        hm.hybrid_moe_forward_stage(layer, wts[i % copies], x, lg, y, scratch, hm.STAGE_W13)
    k1.record()
    torch.cuda.synchronize()
    w13_launch_us = k0.elapsed_time(k1) * 1e3 / reps

    # the single-launch decode alone (M <= 8 on layers that have it): back-to-back
    # forwards, each one launch, between two events on the launch stream
    fused = bool(hm.moe_layer_query(layer)["fused_decode"]) and w.M <= hm.DECODE_MAX_M
    fused_launch_us = None
    if fused:
        torch.cuda.synchronize()
        torch.cuda._sleep(int(1e8))
        k0.record()
        for i in range(reps):
            hm.hybrid_moe_forward(layer, wts[i % copies], x, lg, y, scratch)
        k1.record()
        torch.cuda.synchronize()
        fused_launch_us = k0.elapsed_time(k1) * 1e3 / reps

    # algorithmic work from the routing this batch produced
    eb = expert_bytes(packed)
    k, M = w.top_k, w.M
    res = {"ms_per_step": ms_per_step, "stage_us": stage_us, "copies": copies, "block_m": block_m,
           "w13_launch_us": w13_launch_us, "fused_launch_us": fused_launch_us,
           "layer_bytes_resident": layer_bytes, "desc": describe(w, packed)}
    io_bytes = M * w.H * 2 + M * w.E * 4 + M * w.H * 2        # x, logits, y
    flops = 6.0 * M * k * w.H * w.I
    res["act_format"] = act_format
    if M <= hm.DECODE_MAX_M and not act_format:
        v = hm.moe_decode_view(layer, scratch)
        counts = v["counts"].cpu().numpy()
        nd, nk = int(counts[0]), int(counts[1])
        n_tier = {"kept": nk, "nf3": nd - nk}
        w13 = sum(n_tier[t] * eb[t]["w13"] for t in eb)
        w2 = sum(n_tier[t] * eb[t]["w2"] for t in eb)
        # W13 GEMV: the touched experts' W13, x read, h written (fp32)
        res.update(distinct_experts=nd, distinct_kept=nk, touched_experts=n_tier,
                   layer_bytes=w13 + w2 + io_bytes,
                   w13_bytes=w13 + M * w.H * 2 + M * k * w.I * 4)
    else:
        touched = {}
        for t, name in ((0, "kept"), (1, "nf3")):
            if name not in eb:
                continue
            off = hm.moe_align_view(layer, scratch, t)["expert_off"].cpu().numpy()
            touched[name] = int((np.diff(off) > 0).sum())
        wbytes = sum(touched[t] * (eb[t]["w13"] + eb[t]["w2"]) for t in touched)
        w13w = sum(touched[t] * eb[t]["w13"] for t in touched)
        # W13 grouped GEMM: the touched experts' W13, the fp16 x read, h written (fp16)
        res.update(touched_experts=touched, layer_bytes=wbytes + io_bytes,
                   w13_bytes=w13w + M * w.H * 2 + M * k * w.I * 2)
    res.update(flops=flops, w13_flops=4.0 * M * k * w.H * w.I)
    res["packed"] = packed
    res["inputs"] = (synth.activations_bf16(w, w.M), synth.router_logits(w, w.M))
    del graphs, wts, base
    torch.cuda.empty_cache()
    return res


def rocprof_launch_us(kernel_key, src_hash):
    """Average duration (us) of a workload's dominant kernel in the committed rocprofv3
    kernel trace (profiles/kernel_times.json), if it was taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None, None
    if not rec or rec.get("source_hash") != src_hash:
        return None, None
    return float(rec["avg_us"]), rec.get("profile")


def roofline(w, r, src, decode):
    """Roofline of the dominant kernel: the single-launch decode kernel (the whole
    step: every algorithmic byte of the layer) where the layer has it, else the W13
    stage. The bound follows the layer's arithmetic intensity (flops per algorithmic
    byte) against the ridge point of the peaks."""
    intensity = r["flops"] / r["layer_bytes"]
    hbm = decode or intensity < RIDGE_FLOP_PER_BYTE
    fused = decode and r.get("fused_launch_us") is not None
    w4a4 = bool(r.get("act_format"))
    key = ("decode_fused_" if fused else "decode_w13_" if decode else
           "w4a4_w13_" if w4a4 else "prefill_w13_") + w.name
    if fused:
        work, scale, peak, unit = r["layer_bytes"], 1e9, HBM_PEAK_GBPS, "GB/s"
    elif hbm:
        work, scale, peak, unit = r["w13_bytes"], 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        work, scale, peak, unit = r["w13_flops"], 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    kernel = ("decode_fused_kernel (the whole decode forward)" if fused
              else "w13_gemv_kernel (decode W13 + SwiGLU)" if decode
              else "W13 stage: mx_gemm_kernel<W13> (kept tier, W4A4) + grouped_gemm_kernel<W13> "
                   "(NF3 tier) + h quantiser" if w4a4
              else "grouped_gemm_kernel<W13> (prefill W13 + SwiGLU)")
    ev_us = r["fused_launch_us"] if fused else r["w13_launch_us"]
    prof_us, prof = rocprof_launch_us(key, src)
    us = prof_us if prof_us is not None else ev_us
    achieved = work / (us * 1e-6) / scale
    rec = {"bound": "hbm" if hbm else "mfma", "kernel": kernel, "achieved": achieved, "peak": peak,
           "unit": unit, "frac": achieved / peak,
           "traffic": pmc_traffic(key, src, None),
           ("algorithmic_bytes" if hbm else "algorithmic_flops"): work,
           "avg_launch_us": us,
           "timing": "rocprofv3 kernel trace" if prof_us is not None else "hip events",
           "profile": prof,
           "avg_launch_us_hip_events": ev_us,
           "achieved_hip_events": work / (ev_us * 1e-6) / scale,
           "frac_hip_events": work / (ev_us * 1e-6) / scale / peak,
           "intensity_flop_per_byte": intensity}
    return rec


def cpu_baseline(packed, x_bits, logits, runs, tokens=None):
    """The oracle as it stands on the same layer and batch (or on a sample of its tokens,
    routed with the whole batch): `runs` forwards, the median reported."""
    from oracle import layer as OL
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        pass
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        OL.forward(packed, x_bits, logits, tokens=tokens)
        times.append(time.perf_counter() - t0)
    med = sorted(times)[len(times) // 2]
    M = x_bits.shape[0]
    n = M if tokens is None else len(tokens)
    what = f"the whole M={M} batch" if tokens is None else f"{n} of the M={M} tokens (routing all {M})"
    try:
        nproc = len(os.sched_getaffinity(0))
    except Exception:
        nproc = os.cpu_count()
    return {"value": n / med, "unit": "tok/s", "cores": blas or 1, "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "nproc": nproc, "blas_threads": blas,
            "runs": runs, "median_s": med, "run_s": times,
            "sample": f"median of {runs} oracle forwards of {what}: route, fp32 dequant of the "
                      f"touched experts, fp64 SwiGLU MLPs, combine; numpy, matmuls on "
                      f"{blas} BLAS threads (`cores`), elementwise work single-threaded"}


def workload_record(w, r, decode, args, steps):
    """The fields one workload contributes to the JSON line."""
    ms = r["ms_per_step"]
    src = source_hash(*kernel_sources(decode, bool(r.get("act_format"))))
    rec = {"workload": r["desc"], "M": w.M, "ms_per_step": ms, "tok_per_s": w.M / (ms * 1e-3),
           "steps": steps, "weight_copies_rotated": r["copies"],
           "hbm_gbps": r["layer_bytes"] / (ms * 1e-3) / 1e9,
           "hbm_frac_layer": r["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "tflops": r["flops"] / (ms * 1e-3) / 1e12,
           "mfma_frac_layer": r["flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "layer_bytes_per_step": r["layer_bytes"], "flops_per_step": r["flops"],
           "touched_experts": r["touched_experts"],
           "stage_us": dict(zip(["route", "w13", "w2", "combine"], [round(v, 2) for v in r["stage_us"]])),
           "roofline": roofline(w, r, src, decode)}
    if not decode:
        rec["block_m"] = r["block_m"]
    if r.get("act_format"):
        rec["activations"] = "kept tier MXFP4 (W4A4), NF3 tail bf16/fp16 (W4A16)"
    return rec


def repack_bench(steps: int, warmup: int) -> dict:
    """Times moe_repack (load-time demux of checkpoint-style per-expert tensors into the
    tier-local arrays, NF3 code planes to the 3-bit stream) on the GLM-class layer with
    random code bytes (a bit shuffle: its speed does not depend on the values)."""
    import numpy as np
    import torch
    import synth
    import weight_only_quantized_moe_amd as hm
    w = synth.glm_decode()
    bm = synth.bit_map(w)
    E, H, I = w.E, w.H, w.I
    layer = hm.moe_layer_create(E, H, I, w.top_k, 8, hm.KEPT_NVFP4, bm, 0)
    g = torch.Generator(device="cuda").manual_seed(0)

    def rnd(n, dtype=torch.uint8):
        return torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda", generator=g).view(dtype)

    experts, src_bytes = [], 0
    for e in range(E):
        if bm[e] == 4:
            ex = {"w13_q": rnd(2 * I * H // 2), "w13_s": rnd(2 * I * H // 16),
                  "w13_g": torch.ones(1, dtype=torch.float32, device="cuda"),
                  "w2_q": rnd(H * I // 2), "w2_s": rnd(H * I // 16),
                  "w2_g": torch.ones(1, dtype=torch.float32, device="cuda")}
        else:
            ex = {"w13_lo": rnd(2 * I * H // 4), "w13_hi": rnd(2 * I * H // 8),
                  "w13_s": rnd(2 * I * H // 32).view(torch.int16),
                  "w2_lo": rnd(H * I // 4), "w2_hi": rnd(H * I // 8),
                  "w2_s": rnd(H * I // 32).view(torch.int16)}
        src_bytes += sum(t.numel() * t.element_size() for t in ex.values())
        experts.append(ex)
    empty = synth.empty_packed_layer(E, H, I, w.top_k, "nvfp4", bm)
    dst = hm.DeviceWeights.__new__(hm.DeviceWeights)
    dst.tensors = {}
    for tier, keys in hm.DeviceWeights.KEYS.items():
        for k in keys:
            a = empty[tier][k]
            dt = torch.int16 if a.dtype == np.uint16 else (torch.float32 if a.dtype == np.float32 else torch.uint8)
            dst.tensors[f"{tier}_{k}"] = None if a.size == 0 else torch.empty(a.shape, dtype=dt, device="cuda")
    dst._rebuild()
    dst_bytes = dst.nbytes()
    for _ in range(warmup):
        hm.moe_repack(layer, experts, dst)
    torch.cuda.synchronize()
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        hm.moe_repack(layer, experts, dst)
    t.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(t) / steps
    moved = src_bytes + dst_bytes
    gbps = moved / (ms * 1e-3) / 1e9
    return {"metric": "moe_repack GB/s (load-time demux + NF3 repack, bytes read + written)",
            "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "u8", "data": "synthetic",
            "config": {"workload": f"repack {describe(w, empty)}", "bytes_read": src_bytes,
                       "bytes_written": dst_bytes},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "traffic": None}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None,
                    choices=["qwen_decode", "glm_decode", "glm_prefill", "glm_mxfp4", "glm_uniform"],
                    help="run this workload alone (default: Qwen-shaped decode M=8 with its sweep, "
                         "and GLM-class prefill M=4096)")
    ap.add_argument("--m", type=int, default=None, help="override the batch size")
    ap.add_argument("--w4a4", action="store_true",
                    help="with --workload glm_mxfp4: the kept tier as W4A4 (MXFP4 activations)")
    ap.add_argument("--copies", type=int, default=None, help="weight copies to rotate")
    ap.add_argument("--no-sweep", action="store_true", help="skip the M=1,2,4 decode sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=None, metavar="MIB",
                    help="only copy MIB mebibytes device to device five times (the plain copy "
                         "the HBM traffic counters are scaled by) and exit")
    ap.add_argument("--block-m", type=int, default=None,
                    help="prefill GEMM rows per expert block (16/32/64/128; default: the library picks "
                         "from max_tokens * top_k / E)")
    ap.add_argument("--repack", action="store_true",
                    help="time the load-time demux/repack (moe_repack) of the GLM-class layer "
                         "instead of a forward")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the hybrid MoE layer "
                                   "is measured on one MI355X with the full layer resident; "
                                   "multi-GPU sharding is not implemented (see DESIGN.md)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.repack:
        print(json.dumps(repack_bench(min(args.steps, 20), min(args.warmup, 2))))
        return
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}))
        return
    import weight_only_quantized_moe_amd as hm
    hm.load_library()

    default = args.workload is None
    w = workload(args.workload or "qwen_decode", args.m)
    decode = w.M <= hm.DECODE_MAX_M
    log(f"measuring {w.name} (M={w.M}), {args.steps} steps after {args.warmup} warm-up")
    r = measure(w, args.steps, args.warmup, args.copies, block_m=args.block_m,
                act_format=1 if args.w4a4 else 0)
    rec = workload_record(w, r, decode, args, args.steps)
    ms = r["ms_per_step"]
    out = {
        "metric": METRIC,
        "value": w.M / (ms * 1e-3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["desc"], "M": w.M, "tokens_per_step": w.M,
                   "weight_copies_rotated": r["copies"], "launch": "hip_graph_replay",
                   "parallelism": "single_gpu"},
        "hbm_gbps": rec["hbm_gbps"],
        "hbm_frac_layer": rec["hbm_frac_layer"],
        "layer_bytes_per_step": rec["layer_bytes_per_step"],
        "stage_us": rec["stage_us"],
        "roofline": rec["roofline"],
    }
    if decode:
        out["config"]["distinct_experts"] = r["distinct_experts"]
    else:
        out["tflops"] = rec["tflops"]
        out["mfma_frac_layer"] = rec["mfma_frac_layer"]
        out["config"]["touched_experts"] = r["touched_experts"]
        out["config"]["block_m"] = r["block_m"]
    if decode:
        # the same batch with the decode forward as one persistent launch
        rs = measure(w, args.steps, args.warmup, args.copies, packed=r["packed"], decode_launch=1)
        out["single_launch"] = {
            "kernel": "decode_fused_kernel (routing, W13 + SwiGLU, W2, combine in one launch)",
            "ms_per_step": rs["ms_per_step"], "tok_per_s": w.M / (rs["ms_per_step"] * 1e-3),
            "hbm_frac_layer": rs["layer_bytes"] / (rs["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "avg_launch_us_hip_events": rs["fused_launch_us"],
            "default_ms_per_step": ms}
    if decode and w.name.startswith("qwen_decode") and not args.no_sweep and args.m is None:
        sweep = []
        for m in (1, 2, 4):
            wm = workload("qwen_decode", m)
            rm = measure(wm, args.steps, args.warmup, args.copies, packed=r["packed"])
            rr = workload_record(wm, rm, True, args, args.steps)
            sweep.append({"M": m, "tok_per_s": rr["tok_per_s"], "ms_per_step": rr["ms_per_step"],
                          "hbm_gbps": rr["hbm_gbps"], "hbm_frac_layer": rr["hbm_frac_layer"],
                          "w13_frac_of_hbm_peak": rr["roofline"]["frac_hip_events"],
                          "distinct_experts": rm["distinct_experts"]})
        sweep.append({"M": w.M, "tok_per_s": out["value"], "ms_per_step": ms, "hbm_gbps": out["hbm_gbps"],
                      "hbm_frac_layer": out["hbm_frac_layer"],
                      "w13_frac_of_hbm_peak": out["roofline"]["frac_hip_events"],
                      "distinct_experts": r["distinct_experts"]})
        out["sweep"] = sweep
    if not args.no_cpu_baseline:
        x_bits, logits = r["inputs"]
        log("timing the CPU oracle")
        cb = cpu_baseline(r["packed"], x_bits, logits, 5 if decode else 3,
                          tokens=None if decode else [0])
        if not decode:
            cb["value_tflops"] = r["flops"] * cb["value"] / w.M / 1e12
        out["cpu_baseline"] = cb
    del r
    if default:
        # the prefill half of the metric: the GLM-class layer at M = 4096
        wp = workload("glm_prefill", None)
        psteps = max(5, min(args.steps, 100))
        log(f"measuring {wp.name} (M={wp.M}), {psteps} steps after {min(args.warmup, 10)} warm-up")
        rp = measure(wp, psteps, min(args.warmup, 10), args.copies)
        prec = workload_record(wp, rp, False, args, psteps)
        if not args.no_cpu_baseline:
            x_bits, logits = rp["inputs"]
            log("timing the CPU oracle (prefill sample)")
            cb = cpu_baseline(rp["packed"], x_bits, logits, 3, tokens=[0])
            cb["value_tflops"] = rp["flops"] * cb["value"] / wp.M / 1e12
            prec["cpu_baseline"] = cb
        out["prefill"] = prec
        del rp
        # the W4A4 kept tier (MXFP4 weights and activations on MX-scaled matrix cores) on
        # the GLM-class MXFP4 + NF3 layer at M = 512, beside the same layer as W4A16
        wx = workload("glm_mxfp4", None)
        log(f"measuring {wx.name} (M={wx.M}) W4A4 and W4A16")
        rx = measure(wx, psteps, min(args.warmup, 10), args.copies, act_format=1)
        xrec = workload_record(wx, rx, False, args, psteps)
        r16 = measure(wx, psteps, min(args.warmup, 10), args.copies, packed=rx["packed"])
        xrec["w4a16_same_layer"] = {"ms_per_step": r16["ms_per_step"],
                                    "tok_per_s": wx.M / (r16["ms_per_step"] * 1e-3),
                                    "stage_us": dict(zip(["route", "w13", "w2", "combine"],
                                                         [round(v, 2) for v in r16["stage_us"]]))}
        out["w4a4"] = xrec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
