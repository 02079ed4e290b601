"""Benchmark of the fused multi-tenant LoRA layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_qkv] [--sets S] [--act mxfp8|bf16]

(``--workload decoder_layer``: a step is one decoder layer's four LoRA projections chained on
one segment build; see ``decoder_layer``.)

A step is one pass of the whole hot path over one batch: one fused layer call
(gemm_lowp_lora_epilogue with LORA_FUSE_SHRINK | LORA_BUILD_SEGMENTS: the segment builder,
the down-projection and the GEMM with its LoRA epilogue in one launch; above 16 tokens
also the MXFP8 pre-pass launch), from bf16 x and adapter ids to bf16 y.  The K timed steps are captured in one HIP graph and replayed once,
bracketed by torch.cuda.synchronize(); inputs are resident in HBM.  Steps rotate over S
copies of the inputs so that the weights are read from HBM rather than from the 256 MB
Infinity Cache.  ``--act bf16`` times the 16-bit activation variant (LORA_ACT_BF16: x
enters the base product in bf16, W widened to bf16).

Printed: one JSON line with the metric, the roofline of the dominant kernel (the fused
layer kernel: algorithmic bytes or FLOPs per call over its average duration, timed with
HIP events around a graph of K layer calls on the launch stream) and the oracle's CPU
time on a bounded sample (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per fused LoRA-layer call and achieved HBM TB/s (decode) / MFMA TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0     # dense FP8 (and FP8 x FP4) MFMA, MI355X
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA, MI355X (the 16-bit activation variant)
CSRC = os.path.join(ROOT, "precision_gemm_amd", "csrc")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(wl):
    """Algorithmic bytes and FLOPs of one layer call: x, W (codes + scales), A_a and B_a
    of every adapter present (once each), y; 2TKN + sum_tokens 2 r_a (K + N)."""
    present = np.unique(wl.ids)
    ab = sum(int(wl.A[a].size + wl.B[a].size) * 2 for a in present)
    nbytes = wl.x.size * 2 + wl.w_q.nbytes + wl.w_scale.nbytes + ab + wl.T * wl.N * 2
    r_tok = wl.ranks[np.asarray(wl.ids)]
    flops = 2.0 * wl.T * wl.K * wl.N + float(np.sum(2.0 * r_tok * (wl.K + wl.N)))
    return int(nbytes), flops


def cpu_baseline(wl, budget_s: float = 12.0, act: str = "mxfp8"):
    """The oracle as it stands, timed on the host on a bounded sample of the workload."""
    from oracle.layer import LowpWeight, layer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    w = LowpWeight(wl.fmt, wl.w_q, wl.w_scale)
    # sample: whole layer for decode shapes; a slice of tokens for the prefill shape
    rows = np.arange(wl.T) if wl.T <= 256 else np.linspace(0, wl.T - 1, 256).astype(int)
    runs, t0 = 0, time.perf_counter()
    while True:
        layer(wl.x[rows], w, wl.A, wl.B, wl.scale, np.asarray(wl.ids)[rows], act=act)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    per_call = el / runs * (wl.T / len(rows))      # scaled to one whole layer call
    sample = (f"{runs} oracle run(s) of the whole layer" if len(rows) == wl.T else
              f"{runs} oracle run(s) on {len(rows)} of {wl.T} tokens, scaled by T/{len(rows)}")
    return {"value": per_call * 1e6, "unit": "us/call", "cores": int(cores), "kind": "oracle",
            "sample": sample + f" ({el:.1f} s)"}


# one decoder layer's LoRA projections (Llama-3-8B shapes), 16-token decode, 8 adapters
DECODER_LAYER = [("qkv", 4096, 6144, "fp8"), ("o", 4096, 4096, "fp8"), ("gate_up", 4096, 28672, "fp8"),
                 ("down", 14336, 4096, "mxfp4")]
DECODER_RANKS = [8, 16, 16, 32, 64, 8, 16, 32]


def decoder_layer(args):
    """A step is the four projections of one decoder layer chained on one segment build
    (the first call builds the segments in its launch, the others read them)."""
    import torch
    import precision_gemm_amd as P
    import workloads
    from workloads.device import upload
    from oracle.layer import LowpWeight, layer
    a16 = args.act == "bf16"
    T = 16
    ids = np.random.default_rng(60).integers(0, len(DECODER_RANKS), T)
    wls = [workloads.make_custom(T, K, N, fmt, DECODER_RANKS, ids, [1.0 + 0.25 * a for a in range(len(DECODER_RANKS))],
                                 61 + i, name=name, b_std=0.02) for i, (name, K, N, fmt) in enumerate(DECODER_LAYER)]
    nbytes = sum(algorithmic(wl)[0] for wl in wls)
    flops = sum(algorithmic(wl)[1] for wl in wls)
    sets = args.sets or max(1, min(32, int(np.ceil(2 * 256e6 / nbytes)) + 1))
    print(f"[bench] uploading {sets} input set(s) of {nbytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    S = []
    for _ in range(sets):
        ids_d = torch.from_numpy(np.asarray(ids, np.int32)).cuda()
        seg = P.empty_segments(ids_d, len(DECODER_RANKS))
        projs = []
        for wl in wls:
            x, w, ad, _ = upload(wl)
            projs.append(dict(x=x, w=w, ad=ad, ws=P.alloc_workspace(T, wl.K, wl.N, ad.n, ad.r_max),
                              y=torch.empty((T, wl.N), dtype=torch.bfloat16, device="cuda")))
        S.append(dict(seg=seg, projs=projs))
    torch.cuda.synchronize()

    def step(s):
        d = S[s % sets]
        for i, q in enumerate(d["projs"]):
            P.gemm_lowp_lora_epilogue(q["x"], q["w"], d["seg"], q["ad"], q["ws"], fuse_shrink=True, y=q["y"],
                                      build_segments=(i == 0), act_bf16=a16)

    step(0)
    torch.cuda.synchronize()
    worst = {"max_rel": 0.0, "frob_rel": 0.0}
    for wl, q in zip(wls, S[0]["projs"]):
        ref = layer(wl.x, LowpWeight(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale, wl.ids, act=args.act)["y"]
        dlt = q["y"].float().cpu().numpy().astype(np.float64) - ref
        worst["max_rel"] = max(worst["max_rel"], float(np.abs(dlt).max() / np.abs(ref).max()))
        worst["frob_rel"] = max(worst["frob_rel"], float(np.linalg.norm(dlt) / np.linalg.norm(ref)))
    parity = dict(worst, rows_checked=T, projections=len(wls),
                  **{"pass": worst["max_rel"] <= 1e-2 and worst["frob_rel"] <= 5e-3})
    for i in range(args.warmup):
        step(i)
    K = args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / K
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ev_us = e0.elapsed_time(e1) * 1e3 / K
    status = max(P.workspace_status(q["ws"]) for d in S for q in d["projs"])
    achieved = nbytes / (ev_us * 1e-6) / 1e9
    out = {
        "metric": METRIC, "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16xfp8" if a16 else "fp8", "data": "synthetic",
        "config": {"workload": "decoder_layer", "activations": args.act, "T": T,
                   "projections": [f"{n}: K={k} N={m} {f}" for n, k, m, f in DECODER_LAYER],
                   "adapters": len(DECODER_RANKS), "ranks": sorted(set(DECODER_RANKS)), "input_sets": sets,
                   "timing": "hip graph of K steps (four layer calls each)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "k_layer x 4 (the chain's four launches together)", "per_call_bytes": nbytes,
                     "per_call_flops": flops, "kernel_us": ev_us},
        "parity": parity, "device_status": status, "kernel_sha": kernel_source_sha(),
    }
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        parts = [cpu_baseline(wl, budget_s=4.0, act=args.act) for wl in wls]
        out["cpu_baseline"] = {"value": sum(p["value"] for p in parts), "unit": "us/call",
                               "cores": max(p["cores"] for p in parts), "kind": "oracle",
                               "sample": "the four projections, each: " + "; ".join(p["sample"] for p in parts)}
    print(json.dumps(out))


def stored_traffic(workload: str, sha: str):
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sha") != sha:
        return None
    return d.get("hbm_bytes_per_call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_qkv",
                    choices=["tiny", "decode_qkv", "decode_gateup", "prefill", "downproj_fp4", "decoder_layer"])
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0: enough for 2x 256 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--act", choices=["mxfp8", "bf16"], default="mxfp8",
                    help="activations of the base product: MXFP8 (default) or bf16 as they are")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after the timed region, run three plain device copies of this many MiB (untimed): "
                         "the reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU only; --gpus must be 1 "
                          "(sharding across GPUs is not implemented)"}))
        sys.exit(2)

    import torch
    import precision_gemm_amd as P
    import workloads
    from workloads.device import upload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "decoder_layer":
        decoder_layer(args)
        return
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    wl = workloads.make(args.workload)
    a16 = args.act == "bf16"
    nbytes, flops = algorithmic(wl)
    sets = args.sets or max(1, min(32, int(np.ceil(2 * 256e6 / nbytes)) + 1))
    print(f"[bench] uploading {sets} input set(s) of {nbytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    S = []
    for _ in range(sets):
        x, w, ad, ids = upload(wl, dev)
        ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max, dev)
        y = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device=dev)
        seg = P.empty_segments(ids, ad.n)
        S.append(dict(x=x, w=w, ad=ad, ids=ids, ws=ws, y=y, seg=seg))
    torch.cuda.synchronize()

    def step(s):
        d = S[s % sets]
        P.gemm_lowp_lora_epilogue(d["x"], d["w"], d["seg"], d["ad"], d["ws"], fuse_shrink=True, y=d["y"],
                                  build_segments=True, act_bf16=a16)

    # The layer kernel as the step launches it: up to 128 tokens the segment builder is a
    # workgroup of that launch; above, the call launches the builder first, and the layer
    # kernel alone is the call without the flag (the segments are built by then).
    in_launch = wl.T <= 128
    # (the 16-bit activation variant has no MXFP8 pre-pass)
    xq_pass = (not a16) and bool(P.plan_info(wl.T, wl.K, wl.N, S[0]["ad"].n, S[0]["ad"].r_max, wl.fmt)["XQ"])

    def layer_call(s):
        d = S[s % sets]
        P.gemm_lowp_lora_epilogue(d["x"], d["w"], d["seg"], d["ad"], d["ws"], fuse_shrink=True, y=d["y"],
                                  build_segments=in_launch, act_bf16=a16)

    def quant_call(s):  # the MXFP8 pre-pass that the call runs before the layer kernel
        P.quant_act_mxfp8(S[s % sets]["x"])

    # parity of the benchmarked call against the oracle (whole layer for decode shapes)
    step(0)
    torch.cuda.synchronize()
    parity = None
    try:
        from oracle.layer import LowpWeight, layer
        rows = np.arange(wl.T) if wl.T <= 256 else np.linspace(0, wl.T - 1, 128).astype(int)
        ref = layer(wl.x[rows], LowpWeight(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale, np.asarray(wl.ids)[rows],
                    act=args.act)
        yg = S[0]["y"].float().cpu().numpy().astype(np.float64)[rows]
        dlt = yg - ref["y"]
        parity = {"max_rel": float(np.abs(dlt).max() / np.abs(ref["y"]).max()),
                  "frob_rel": float(np.linalg.norm(dlt) / np.linalg.norm(ref["y"])),
                  "rows_checked": int(len(rows)),
                  "pass": bool(np.abs(dlt).max() <= 1e-2 * np.abs(ref["y"]).max()
                               and np.linalg.norm(dlt) <= 5e-3 * np.linalg.norm(ref["y"]))}
    except Exception as e:  # pragma: no cover
        parity = {"error": repr(e)}

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    K = args.steps
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i)
        torch.cuda.synchronize()
        total_s = time.perf_counter() - t0
        layer_us = quant_us = None
    else:
        # K whole steps in one graph, timed from the host
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for i in range(K):
                step(i)
        # K layer calls, timed with events on the launch stream: the layer kernel's
        # duration including its launch gap (with the pre-pass where the plan has one,
        # whose own graph below is subtracted)
        g_layer = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_layer):
            for i in range(K):
                layer_call(i)
        g_quant = None
        if xq_pass:
            g_quant = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_quant):
                for i in range(K):
                    quant_call(i)
        g_all.replay()
        g_layer.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_all.replay()
        torch.cuda.synchronize()
        total_s = time.perf_counter() - t0

        def event_us(g):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / K

        layer_us = event_us(g_layer)
        quant_us = event_us(g_quant) if g_quant is not None else 0.0
        layer_us -= quant_us
    # every workspace must report a clean status
    status = max(P.workspace_status(d["ws"]) for d in S)

    us_per_step = total_s * 1e6 / K
    dom_us = layer_us if layer_us is not None else us_per_step
    prefill = wl.T > 256
    if prefill:
        achieved = flops / (dom_us * 1e-6) / 1e12
        peak = BF16_PEAK_TFLOPS if a16 else FP8_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    else:
        achieved = nbytes / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    sha = kernel_source_sha()
    tag = args.workload + ("_act_bf16" if a16 else "")
    roof["traffic"] = stored_traffic(tag, sha)
    roof["kernel"] = ("k_layer (fused down-projection + bf16-MFMA GEMM on widened W + LoRA epilogue)" if a16 else
                      "k_layer (fused down-projection + scaled-MFMA GEMM + LoRA epilogue)")
    roof["per_call_bytes"] = nbytes
    roof["per_call_flops"] = flops
    roof["kernel_us"] = dom_us

    out = {
        "metric": METRIC,
        "value": round(us_per_step, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": us_per_step / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16xfp8" if wl.fmt == "fp8" else "bf16xfp4") if a16 else ("fp8" if wl.fmt == "fp8" else "fp8xfp4"),
        "data": "synthetic",
        "config": {"workload": args.workload, "activations": args.act, "T": wl.T, "K": wl.K, "N": wl.N, "w_format": wl.fmt,
                   "adapters": wl.n_adapters, "adapters_present": int(len(np.unique(wl.ids))),
                   "ranks": sorted(set(int(r) for r in wl.ranks)), "seed": wl.seed, "input_sets": sets,
                   "timing": "eager" if args.eager else "hip graph of K steps"},
        "roofline": roof,
        "layer_us": layer_us,
        "prepass_us": quant_us,
        "tbps": nbytes / (dom_us * 1e-6) / 1e12,
        "tflops": flops / (dom_us * 1e-6) / 1e12,
        "parity": parity,
        "device_status": status,
        "kernel_sha": sha,
    }
    if args.copy_mb > 0:
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, act=args.act)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
