#!/usr/bin/env python3
"""Benchmark of one MoE expert layer (route -> permute -> FC1+act+requant -> FC2 -> combine)
on one MI355X, through the C ABI.  Prints ONE JSON line.

A step is one moe_layer call over one batch of synthetic input already resident in HBM.
The expert weights rotate over enough copies that their working set exceeds the 256 MB
Infinity Cache, so weight bytes come from HBM.  The dominant kernel's average duration
is measured with HIP events on the launch stream; its algorithmic bytes / FLOPs give the
roofline fraction.  The CPU oracle is timed on a bounded sample of the same workload.
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


# the translation unit of the FC1 kernel: the HBM traffic counters stay valid while these are unchanged
FC1_SOURCES = ("grouped_gemm.hip", "device_common.hpp", "moe_internal.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for name in FC1_SOURCES:
        h.update(open(os.path.join(ROOT, "moe_expert_layer_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(w, R, active, counts):
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


def cpu_baseline(w, inp, budget_s=20.0):
    """Time the oracle as it stands on a bounded token sample (about budget_s of work)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    n = min(w.tokens, 16)
    spent, toks = 0.0, 0
    rng = np.random.default_rng(0)
    while True:
        sample = np.sort(rng.choice(w.tokens, size=n, replace=False))
        t0 = time.perf_counter()
        O.layer_tokens(w, inp, sample)
        dt = time.perf_counter() - t0
        spent, toks = spent + dt, toks + n
        if spent >= budget_s / 2 or n == w.tokens:
            break
        n = min(w.tokens, max(n + 1, int(n * min(4.0, (budget_s / 2 - spent) / max(dt, 1e-3)))))
    return {"value": toks / spent, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{toks} tokens of workload {w.name} (oracle.layer_tokens: full routing + FFN of the sampled "
                      f"tokens' rows), {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="oai", help="workload name or index (tiny, oai, decode, prefill_zipf, "
                                                     "mxfp4_large)")
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--weights", choices=["fp8", "fp8e5m2", "mxfp4", "bf16"], default=None,
                    help="replace the workload's weight format (FP8 E4M3, FP8 E5M2, MXFP4, or the BF16 layer)")
    ap.add_argument("--shared", type=int, default=0, help="shared experts (every token, weight 1)")
    ap.add_argument("--scaling", choices=["block", "tensor"], default="block",
                    help="blockwise UE8M0 scales, or one float32 scale per tensor (FP8 weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-steps", type=int, default=20, help="timed launches of the dominant kernel")
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
    cfg = int(args.config) if args.config.isdigit() else args.config
    w = synth.workload(cfg)
    if args.weights and args.weights != w.weight_format:
        w = synth.shrink(w, weight_format=args.weights, name=f"{w.name}/{args.weights}")
    if args.scaling == "tensor":
        w = synth.tensor_scaled(w, name=f"{w.name}/tensor")
    if args.shared:
        w = synth.shrink(w, num_shared=args.shared, name=f"{w.name}/shared{args.shared}")
    t0 = time.time()
    inp = synth.generate(w)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda() for k, v in inp.items()}
    d = B.desc_from_workload(w, args.variant)
    ws = B.alloc_workspace(d)
    T, k, EL = w.tokens, w.topk, w.num_local
    y = torch.empty((T, w.hidden), dtype=torch.int16, device="cuda")
    counts = torch.empty(EL, dtype=torch.int32, device="cuda")
    offsets = torch.empty(EL + 1, dtype=torch.int32, device="cuda")
    wbytes = sum(dev[n].numel() for n in ("w1", "w1_sf", "w2", "w2_sf"))
    copies = max(1, -(-512 * 2 ** 20 // wbytes))  # working set of weights > 2x the Infinity Cache
    wsets = [(dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"])]
    for _ in range(copies - 1):
        wsets.append(tuple(t.clone() for t in wsets[0]))
    stream = torch.cuda.current_stream()

    def step(i):
        w1, w1s, w2, w2s = wsets[i % len(wsets)]
        B.moe_layer(d, dev["logits"], dev["x"], dev["x_sf"], w1, w1s, w2, w2s, y, ws, counts=counts,
                    offsets=offsets, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    ms = e0.elapsed_time(e1) / args.steps

    cnt = counts.cpu().numpy()
    S = w.num_shared
    R = int(cnt.sum()) + S * T           # routed rows, then the shared experts' T rows each
    active = int((cnt > 0).sum()) + S    # experts whose weights are read
    alg = algorithmic(w, R, active, cnt)

    # dominant kernel: FC1 grouped GEMM (fused activation + requant), timed alone on the same stream
    r2s = torch.empty(T * k, dtype=torch.int32, device="cuda")
    s2r = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route_permute(d, dev["logits"], ids, tw, counts, offsets, r2s, s2r, ws, stream=stream)
    h_dtype = torch.int16 if w.weight_format == "bf16" else torch.uint8  # BF16 layer: two bytes per value
    h = torch.empty((T * (k + S), w.inter), dtype=h_dtype, device="cuda")
    h_sf = torch.empty((T * (k + S), w.inter // 128), dtype=torch.uint8, device="cuda")
    for i in range(3):
        w1, w1s, _, _ = wsets[i % len(wsets)]
        B.moe_grouped_fc1_swiglu(d, dev["x"], dev["x_sf"], w1, w1s, offsets, r2s, h, h_sf, ws, stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.kernel_steps):
        w1, w1s, _, _ = wsets[i % len(wsets)]
        B.moe_grouped_fc1_swiglu(d, dev["x"], dev["x_sf"], w1, w1s, offsets, r2s, h, h_sf, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fc1_ms = e0.elapsed_time(e1) / args.kernel_steps

    compute_bound = w.tokens >= 2048
    if compute_bound:
        peak = PEAK_BF16_TFLOPS if w.weight_format == "bf16" else PEAK_FP8_TFLOPS
        achieved = alg["fc1_flops"] / (fc1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s"}
    else:
        peak = PEAK_HBM_GBS
        achieved = alg["fc1_bytes"] / (fc1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s"}
    roof["frac"] = round(achieved / peak, 4)
    roof["kernel"] = "grouped_gemm_kernel<FC1> (moe_grouped_fc1_swiglu; the tile plan is derived in the kernel)"
    roof["kernel_ms"] = round(fc1_ms, 4)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"fc1_{w.name}_traffic.json")
    if os.path.exists(tpath):
        tj = json.load(open(tpath))
        if tj.get("source_hash") == source_hash():
            traffic = tj.get("bytes_per_launch")
    roof["traffic"] = traffic

    # input quantisation (bf16 -> E4M3 + 1x128 UE8M0) of this workload's activations, HBM-bound
    dq = B.desc_from_workload(synth.shrink(w, scaling="block"), args.variant)
    xb = torch.randn((T, w.hidden), device="cuda").to(torch.bfloat16)
    xq = torch.empty((T, w.hidden), dtype=torch.uint8, device="cuda")
    xq_sf = torch.empty((T, w.hidden // 128), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        B.moe_quantize_act(dq, xb, xq, xq_sf, stream=stream)
    torch.cuda.synchronize()
    # the launches are captured in a HIP graph: at decode sizes the kernel is shorter than a
    # host-side launch, and the graph replay times the device work alone
    qg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(qg):
        for _ in range(args.kernel_steps):
            B.moe_quantize_act(dq, xb, xq, xq_sf)
    qg.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    qg.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    q_ms = e0.elapsed_time(e1) / args.kernel_steps
    del qg
    q_bytes = T * w.hidden * (2 + 1 + 1 / 128)
    input_quant = {"kernel": "quantize_act_kernel (moe_quantize_act, graph-replayed)", "kernel_ms": round(q_ms, 4),
                   "bytes": int(q_bytes), "achieved": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "peak": PEAK_HBM_GBS, "frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xb, xq, xq_sf

    tflops = alg["flops"] / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": {"mxfp4": "fp8xfp4", "bf16": "bf16"}.get(w.weight_format, "fp8"),
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "hidden": w.hidden, "inter": w.inter,
                   "experts": w.num_experts, "local_experts": EL, "topk": k, "activation": w.activation,
                   "weight_format": w.weight_format, "scaling": w.scaling, "shared_experts": S, "rows": R, "active_experts": active,
                   "parallelism": "one GPU's expert share", "weight_copies": len(wsets)},
        "tflops": round(tflops, 2), "pct_fp8_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "pct_mfma_peak_of_dtype": round(100 * tflops / (PEAK_BF16_TFLOPS if w.weight_format == "bf16"
                                                        else PEAK_FP8_TFLOPS), 2),
        "hbm_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(100 * alg["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "wall_ms_timed_region": round(wall_ms, 2),
        "roofline": roof,
        "input_quant": input_quant,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
