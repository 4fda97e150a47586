#!/usr/bin/env python3
"""Benchmark of the MoE expert layer (route -> permute -> FC1+act+requant -> FC2 -> combine)
on one MI355X, through the C ABI.  Prints ONE JSON line.

A step is one moe_layer call over one batch of synthetic input already resident in HBM.
The headline workload (default: the 32768-token MXFP4 share) gives `value`; the other
graded shares (the 128-token decode share and the 4096-token Zipf prefill share) are run
the same way and reported under "workloads".  Each step is bracketed by its own pair of HIP
events on the launch stream (median, p10 and p90 are reported beside the mean over the
timed region).  The expert weights rotate over enough copies that their working set
exceeds the 256 MB Infinity Cache, so weight bytes come from HBM.

The dominant kernel (the FC1 grouped GEMM) is timed alone with HIP events on the stream it
is launched on; its useful FLOPs (or algorithmic bytes, for the HBM-bound shares) per
launch over that time give the roofline fraction.  Probe kernels measure the achievable
matrix-core rate and HBM read bandwidth on the same GPU, reported beside the published
peaks.  The CPU oracle is timed on a bounded token sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOPS & tokens/s at 128-32768 tok/GPU; % of FP8 MFMA / HBM peak"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published, no sparsity)
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
GRADED = ("mxfp4_large", "decode", "prefill_zipf")

# the translation unit of the FC1 kernel: the HBM traffic counters stay valid while these are unchanged
FC1_SOURCES = ("grouped_gemm.hip", "device_common.hpp", "moe_internal.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in FC1_SOURCES:
        h.update(open(os.path.join(ROOT, "moe_expert_layer_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(w, R, active):
    """Useful FLOPs and bytes of the layer and of FC1 / FC2 for this routing."""
    H, I, T, E = w.hidden, w.inter, w.tokens, w.num_experts
    if w.weight_format == "bf16":  # two bytes per element, no scales
        wb = lambda n, k: n * k * 2.0
    elif w.weight_format != "mxfp4":
        wb = lambda n, k: n * k * (1 + 1 / 16384)
    else:
        wb = lambda n, k: n * k * (0.5 + 1 / 32)
    fl1, fl2 = 4.0 * R * H * I, 2.0 * R * H * I
    eb = (2.0, 0.0) if w.weight_format == "bf16" else (1.0, 1 / 128)  # element bytes, scale bytes per element
    x_bytes = T * H * (eb[0] + eb[1])
    h_bytes = R * I * (eb[0] + eb[1])
    b1 = active * wb(2 * I, H) + x_bytes + h_bytes
    b2 = active * wb(H, I) + h_bytes + R * H * 4
    layer_bytes = active * (wb(2 * I, H) + wb(H, I)) + x_bytes + 2 * T * H + 4 * T * E
    return {"flops": fl1 + fl2, "bytes": layer_bytes, "fc1_flops": fl1, "fc1_bytes": b1, "fc2_flops": fl2,
            "fc2_bytes": b2}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s=20.0):
    """Time the oracle as it stands on a bounded token sample (about budget_s / 2 of work).

    What is timed: oracle.layer_tokens on a sorted random sample of tokens, i.e. routing of
    every token, then for each local expert that a sampled token reaches, that expert's
    weights dequantised to float64 and the float64 FFN of the sampled tokens' rows, the
    requant, and the combine.  The weight dequantisation is repeated in every call, as the
    oracle does it."""
    import numpy as np
    from oracle import moe_oracle as O
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pass
    avail = len(os.sched_getaffinity(0))
    n = min(w.tokens, 2)
    spent, toks, calls = 0.0, 0, 0
    rng = np.random.default_rng(0)
    while True:
        sample = np.sort(rng.choice(w.tokens, size=n, replace=False))
        t0 = time.perf_counter()
        O.layer_tokens(w, inp, sample)
        dt = time.perf_counter() - t0
        spent, toks, calls = spent + dt, toks + n, calls + 1
        if spent >= budget_s / 2 or n == w.tokens:
            break
        n = min(w.tokens, max(n + 1, int(n * min(4.0, (budget_s / 2 - spent) / max(dt, 1e-3)))))
    return {"value": round(toks / spent, 2), "unit": "tokens/s", "cores": threads or avail, "kind": "oracle",
            "host_cores_available": avail, "cpu_model": cpu_model(),
            "sample": f"{toks} tokens of workload {w.name} in {calls} calls of oracle.layer_tokens (routing of all "
                      f"{w.tokens} tokens, then float64 dequantisation of each reached expert's weights and the "
                      f"float64 FFN, requant and combine of the sampled tokens' rows), {spent:.1f} s, numpy/BLAS "
                      f"with {threads or avail} threads"}


def pct(a, b):
    return round(100.0 * a / b, 2)


def run_probes(torch, steps=5):
    """Achievable matrix-core rate (FP8 x FP8 and FP8 x FP4 scaled 32x32x64 MFMA loops), HBM read
    bandwidth (a 4 GiB streaming read) and the per-CU rate of the GEMMs' operand stream (direct
    global-to-LDS loads of 512-row panels, from HBM and from L2-resident panels, one or two 64 KB
    stages in flight), each the best of `steps` timed runs."""
    from moe_expert_layer_amd import probe_binding as PB
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    out = {"compute_units": cus}
    blocks, iters = cus * 2, 20000  # two 4-wave workgroups per CU: two waves per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fp4 in (("mfma_fp8", False), ("mfma_fp8xfp4", True)):
        PB.mfma_loop(blocks, 100, sink, b_fp4=fp4)
        best = None
        for _ in range(steps):
            torch.cuda.synchronize()
            e0.record()
            PB.mfma_loop(blocks, iters, sink, b_fp4=fp4)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        flops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 64
        out[name] = {"tflops": round(flops / (best * 1e-3) / 1e12, 1), "published_tflops": PEAK_FP8_TFLOPS,
                     "frac_of_published": round(flops / (best * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    del sink
    nbytes = 4 * 2 ** 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    blocks = cus * 8
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    PB.hbm_read(src, blocks, sink)
    best = None
    for _ in range(steps):
        torch.cuda.synchronize()
        e0.record()
        PB.hbm_read(src, blocks, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    gbs = nbytes / (best * 1e-3) / 1e9
    out["hbm_read"] = {"gbs": round(gbs, 1), "published_gbs": PEAK_HBM_GBS, "frac_of_published": round(gbs / PEAK_HBM_GBS, 4),
                       "bytes": nbytes}
    del sink
    # the GEMMs' operand stream without arithmetic: one 512-thread workgroup per CU streaming
    # 512-row panels into a two-stage ring of 64 KB LDS stages (per-CU load-path rate)
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    for name, K, panels, passes in (("dma_stream_hbm", 7168, 0, 1), ("dma_stream_l2", 2048, 8, 16)):
        for depth in (1, 2):
            PB.dma_stream(src, K, cus, panels, 1, depth, sink)
            best = None
            for _ in range(steps):
                torch.cuda.synchronize()
                e0.record()
                PB.dma_stream(src, K, cus, panels, passes, depth, sink)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
            moved = cus * passes * 512 * K
            out[f"{name}_depth{depth}"] = {"gbs": round(moved / (best * 1e-3) / 1e9, 1),
                                           "gbs_per_cu": round(moved / (best * 1e-3) / 1e9 / cus, 2),
                                           "bytes_per_clk_per_cu_at_2p4ghz": round(moved / (best * 1e-3) / cus / 2.4e9, 2),
                                           "bytes": moved}
    del src, sink
    torch.cuda.empty_cache()
    return out


def make_workload(synth, name, weights=None, scaling="block", shared=0):
    cfg = int(name) if str(name).isdigit() else name
    w = synth.workload(cfg)
    if weights and weights != w.weight_format:
        w = synth.shrink(w, weight_format=weights, name=f"{w.name}/{weights}")
    if scaling == "tensor":
        w = synth.tensor_scaled(w, name=f"{w.name}/tensor")
    if shared:
        w = synth.shrink(w, num_shared=shared, name=f"{w.name}/shared{shared}")
    return w


def run_workload(w, args, torch, np, B, synth, probes=None, keep_inputs=False):
    """Generate, upload and time one workload; returns (entry, host inputs or None)."""
    t0 = time.time()
    inp = synth.generate(w)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda() for k, v in inp.items()}
    d = B.desc_from_workload(w, args.variant)
    ws = B.alloc_workspace(d)
    T, k, EL, S = w.tokens, w.topk, w.num_local, w.num_shared
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    counts = torch.empty(EL, dtype=torch.int32, device="cuda")
    offsets = torch.empty(EL + 1, dtype=torch.int32, device="cuda")
    wbytes = sum(dev[n].numel() * dev[n].element_size() for n in ("w1", "w1_sf", "w2", "w2_sf"))
    copies = max(1, -(-512 * 2 ** 20 // wbytes))  # working set of weights > 2x the Infinity Cache
    wsets = [(dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"])]
    for _ in range(copies - 1):
        wsets.append(tuple(t.clone() for t in wsets[0]))
    stream = torch.cuda.current_stream()

    def step(i):
        w1, w1s, w2, w2s = wsets[i % len(wsets)]
        B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], w1, w1s, w2, w2s, y, ws, counts=counts,
                    offsets=offsets, stream=stream)

    ms = wall_ms = None
    per_step = []
    if not args.kernels_only:
        for i in range(args.warmup):
            step(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t_wall) * 1e3
        ms = e0.elapsed_time(e1) / args.steps
        per_step = np.array([a.elapsed_time(b) for a, b in ev])

    # rows and active experts of this routing (the routing is the same in every step)
    r2s = torch.empty(T * k, dtype=torch.int32, device="cuda")
    s2r = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route_permute(d, dev["logits"], ids, tw, counts, offsets, r2s, s2r, ws, stream=stream)
    cnt = counts.cpu().numpy()
    R = int(cnt.sum()) + S * T           # routed rows, then the shared experts' T rows each
    active = int((cnt > 0).sum()) + S    # experts whose weights are read
    alg = algorithmic(w, R, active)

    # dominant kernel: FC1 grouped GEMM (fused activation + requant), timed alone on the same stream;
    # then FC2 + combine through their entry point
    h_dtype = torch.int16 if w.weight_format == "bf16" else torch.uint8  # BF16 layer: two bytes per value
    h = torch.empty((T * (k + S), w.inter), dtype=h_dtype, device="cuda")
    h_sf = torch.empty((T * (k + S), w.inter // 128), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def fc1(i):
        w1, w1s, _, _ = wsets[i % len(wsets)]
        B.moe_grouped_fc1_swiglu(d, dev["x"], dev["x_sf"], w1, w1s, offsets, r2s, h, h_sf, ws, stream=stream)

    def fc2(i):
        _, _, w2, w2s = wsets[i % len(wsets)]
        B.moe_grouped_fc2_combine(d, h, h_sf, w2, w2s, offsets, r2s, s2r, tw, y, ws, stream=stream)

    timed = {}
    for name, fn in (("fc1", fc1), ("fc2_combine", fc2)):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.kernel_steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        timed[name] = e0.elapsed_time(e1) / args.kernel_steps
    fc1_ms = timed["fc1"]

    compute_bound = w.tokens >= 2048
    mixed = w.weight_format == "mxfp4"
    if compute_bound:
        peak = PEAK_BF16_TFLOPS if w.weight_format == "bf16" else PEAK_FP8_TFLOPS
        achieved = alg["fc1_flops"] / (fc1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s"}
    else:
        peak = PEAK_HBM_GBS
        achieved = alg["fc1_bytes"] / (fc1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s"}
    roof["frac"] = round(achieved / peak, 4)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"fc1_{w.name}_traffic.json")
    if os.path.exists(tpath):
        tj = json.load(open(tpath))
        if tj.get("source_hash") == source_hash():
            traffic = tj.get("bytes_per_launch")
    roof["traffic"] = traffic
    roof["kernel"] = "grouped_gemm_kernel<FC1> (moe_grouped_fc1_swiglu; the tile plan is derived in the kernel)"
    roof["kernel_ms"] = round(fc1_ms, 4)
    roof["algorithmic_per_launch"] = alg["fc1_flops"] if compute_bound else alg["fc1_bytes"]
    if mixed:
        roof["note"] = "FP8 activations x FP4 weights: the scaled MFMA runs at the FP8 rate with one FP8 operand"
    if probes and compute_bound and "mfma_fp8xfp4" in probes:
        ach = probes["mfma_fp8xfp4" if mixed else "mfma_fp8"]["tflops"]
        roof["frac_of_probe_peak"] = round(achieved / ach, 4)
    elif probes and not compute_bound and "hbm_read" in probes:
        roof["frac_of_probe_peak"] = round(achieved / probes["hbm_read"]["gbs"], 4)

    entry = {"workload": w.name, "tokens": T, "hidden": w.hidden, "inter": w.inter, "experts": w.num_experts,
             "local_experts": EL, "topk": k, "activation": w.activation, "weight_format": w.weight_format,
             "scaling": w.scaling, "shared_experts": S, "rows": R, "active_experts": active,
             "weight_copies": len(wsets), "useful_flops": alg["flops"], "algorithmic_bytes": alg["bytes"]}
    if ms is not None:
        med = float(np.median(per_step))
        p10, p90 = float(np.percentile(per_step, 10)), float(np.percentile(per_step, 90))
        tflops = alg["flops"] / (ms * 1e-3) / 1e12
        entry.update({
            "ms_per_step": round(ms, 4), "ms_median": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "tokens_per_s_median": round(T / (med * 1e-3), 1),
            "tflops": round(tflops, 2), "pct_fp8_peak": pct(tflops, PEAK_FP8_TFLOPS),
            "hbm_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": pct(alg["bytes"] / (ms * 1e-3) / 1e9, PEAK_HBM_GBS),
            "wall_ms_timed_region": round(wall_ms, 2)})
        if probes:
            entry["pct_probe_mfma_peak"] = pct(tflops, probes["mfma_fp8xfp4" if mixed else "mfma_fp8"]["tflops"])
            entry["pct_probe_hbm_peak"] = pct(alg["bytes"] / (ms * 1e-3) / 1e9, probes["hbm_read"]["gbs"])
    entry["roofline"] = roof
    fc2_ms = timed["fc2_combine"]
    entry["fc2_combine"] = {"entry_point": "moe_grouped_fc2_combine (FC2 grouped GEMM + combine kernel)",
                            "ms": round(fc2_ms, 4),
                            "fc2_tflops_incl_combine": round(alg["fc2_flops"] / (fc2_ms * 1e-3) / 1e12, 1)}
    del dev, ws, wsets, h, h_sf, y
    torch.cuda.empty_cache()
    return entry, (inp if keep_inputs else None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mxfp4_large", help="headline workload name or index (tiny, oai, decode, "
                                                             "prefill_zipf, mxfp4_large)")
    ap.add_argument("--also", default=None,
                    help="comma-separated further workloads (default: the other graded shares of decode, "
                         "prefill_zipf, mxfp4_large; 'none' for none)")
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--weights", choices=["fp8", "fp8e5m2", "mxfp4", "bf16"], default=None,
                    help="replace the headline workload's weight format (FP8 E4M3, FP8 E5M2, MXFP4, or the BF16 layer)")
    ap.add_argument("--shared", type=int, default=0, help="shared experts (every token, weight 1)")
    ap.add_argument("--scaling", choices=["block", "tensor"], default="block",
                    help="blockwise UE8M0 scales, or one float32 scale per tensor (FP8 weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the achievable-peak probe kernels")
    ap.add_argument("--kernels-only", action="store_true",
                    help="headline workload only: route/permute once, then the FC1 and FC2+combine entry points "
                         "--kernel-steps times each (a short program for counter collection)")
    ap.add_argument("--kernel-steps", type=int, default=20, help="timed launches of each GEMM entry point")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (reference for the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library computes one GPU's "
              "expert share, and the expert-parallel exchange across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_expert_layer_amd import binding as B
    from moe_expert_layer_amd import synth

    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    probes = None
    if not args.no_probes and not args.kernels_only:
        probes = run_probes(torch)
        print(f"[bench] probes: {json.dumps(probes)}", file=sys.stderr, flush=True)

    head = make_workload(synth, args.config, args.weights, args.scaling, args.shared)
    entry, inp = run_workload(head, args, torch, np, B, synth, probes, keep_inputs=not args.no_cpu_baseline)
    if args.kernels_only:
        print(json.dumps({"kernels_only": head.name, "fc1_ms": entry["roofline"]["kernel_ms"],
                          "fc2_combine_ms": entry["fc2_combine"]["ms"]}), flush=True)
        return
    also = args.also
    if also is None:
        also = [n for n in GRADED if n != head.name]
    elif also == "none":
        also = []
    else:
        also = [a for a in also.split(",") if a]
    others = {}
    for name in also:
        e, _ = run_workload(make_workload(synth, name), args, torch, np, B, synth, probes)
        others[e["workload"]] = e

    mixed = head.weight_format == "mxfp4"
    out = {
        "metric": METRIC, "value": entry["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": entry["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"mxfp4": "fp8xfp4", "bf16": "bf16"}.get(head.weight_format, "fp8"),
        "data": "synthetic",
        "config": {k: entry[k] for k in ("workload", "tokens", "hidden", "inter", "experts", "local_experts", "topk",
                                         "activation", "weight_format", "scaling", "shared_experts", "rows",
                                         "active_experts", "weight_copies")},
    }
    out["config"]["parallelism"] = "one GPU's expert share (32 of 256 experts)" if head.num_experts == 256 else \
        "one GPU's expert share"
    for key in ("ms_median", "ms_p10", "ms_p90", "tokens_per_s_median", "tflops", "pct_fp8_peak", "hbm_gbs",
                "pct_hbm_peak", "pct_probe_mfma_peak", "pct_probe_hbm_peak", "wall_ms_timed_region",
                "useful_flops", "algorithmic_bytes", "fc2_combine"):
        if key in entry:
            out[key] = entry[key]
    if mixed:
        out["pct_fp4_peak"] = pct(entry["tflops"], PEAK_FP4_TFLOPS)
    out["roofline"] = entry["roofline"]
    out["workloads"] = others
    out["probes"] = probes
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(head, inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
