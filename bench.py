"""Benchmark of the fused multi-tenant LoRA layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill] [--sets S] [--act mxfp8|bf16]

(``--workload decoder_layer``: a step is one decoder layer's four LoRA projections chained on
one segment build; see ``decoder_layer``.  ``--backward``: a step is one call of the layer's
backward, lora_backward; see ``backward``.)

A step is one pass of the whole hot path over one batch: one fused layer call
(gemm_lowp_lora_epilogue with LORA_FUSE_SHRINK: the down-projection and the GEMM with its
LoRA epilogue, above 16 tokens after the MXFP8 pre-pass launch, which above 128 tokens also
runs the down-projection), from bf16 x to bf16 y, on a batch whose segments are built (one
build serves every LoRA layer of a step).  The builder alone and the call that builds the
segments too (LORA_BUILD_SEGMENTS) are timed beside it.  The K timed steps are captured in one HIP graph and replayed once,
bracketed by torch.cuda.synchronize(); inputs are resident in HBM.  Steps rotate over S
copies of the inputs so that the weights are read from HBM rather than from the 256 MB
Infinity Cache.  ``--act bf16`` times the 16-bit activation variant (LORA_ACT_BF16: x
enters the base product in bf16, W widened to bf16).

The default workload is the largest single-GPU configuration, the 4096-token multi-tenant
prefill (T = K = N = 4096, FP8 W, 8 adapters of rank 64).

Printed: one JSON line with the metric, the roofline of the layer call (algorithmic bytes
or FLOPs per call over the average duration of the whole call -- MXFP8 pre-pass and layer
kernel -- timed with HIP events around a graph of K calls on the launch stream) and the
oracle's CPU time on a bounded sample (``cpu_baseline``).
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
        if el >= budget_s or runs >= 1000:  # the time budget binds: about 12 s of oracle work
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
    # ablation: the same four projections in the per-token merged-weight formulation
    # (lora_merged_layer, x in bf16), one input set, graph of K steps
    d0 = S[0]
    merged = []
    for wl, q in zip(wls, d0["projs"]):
        wr = P.LowpWeight(wl.fmt, torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda())
        merged.append((q, wr, P.adapter_rows(q["ad"])))
    ids_m = d0["seg"].adapter_id

    def step_merged():
        for q, wr, (rows_, ptrs) in merged:
            P.merged_layer(q["x"], wr, ids_m, q["ad"], ptrs, y=q["y"])

    step_merged()
    gm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gm):
        for i in range(K):
            step_merged()
    gm.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    gm.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    merged_us = e0.elapsed_time(e1) * 1e3 / K
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
        "ablation_merged": {"what": "the four projections as per-token merged-weight layers (lora_merged_layer, "
                                    "x in bf16), us per step", "us": merged_us, "over_fused": merged_us / ev_us},
    }
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        parts = [cpu_baseline(wl, budget_s=4.0, act=args.act) for wl in wls]
        out["cpu_baseline"] = {"value": sum(p["value"] for p in parts), "unit": "us/call",
                               "cores": max(p["cores"] for p in parts), "kind": "oracle",
                               "sample": "the four projections, each: " + "; ".join(p["sample"] for p in parts)}
    print(json.dumps(out))


def tune_shrink(args, wl):
    """The configuration search of the down-projection (precision_gemm_amd.tune) on this
    workload: the library's own configuration against the best one found, microseconds per
    launch of the standalone down-projection."""
    import torch
    import precision_gemm_amd as P
    from precision_gemm_amd import tune
    from workloads.device import upload
    x, w, ad, ids = upload(wl)
    seg = P.build_segments(ids, ad.n)
    torch.cuda.synchronize()
    res = tune.tune_shrink(x, seg, ad, steps=args.tune_shrink, seed=0)
    ref = P.shrink(x, seg, ad)
    best_t = P.shrink_configured(x, seg, ad, tune.to_config(res.best))
    torch.cuda.synchronize()
    names = ("TG", "JP", "U", "TBLK", "ORDER")
    out = {"workload": args.workload, "what": "standalone down-projection, us per launch (HIP events)",
           "start": dict(zip(names, tune.to_config(res.start))), "start_us": res.start_cost,
           "best": dict(zip(names, tune.to_config(res.best))), "best_us": res.best_cost,
           "speedup": res.start_cost / res.best_cost, "steps": len(res.trace), "evaluated": len(res.evaluated),
           "accepted": sum(1 for s in res.trace if s[3]), "t_bitwise_equal": bool(torch.equal(ref, best_t)),
           "trace": [[s[0], dict(zip(names, tune.to_config(s[1]))), round(s[2], 3), s[3]] for s in res.trace],
           "kernel_sha": kernel_source_sha()}
    print(json.dumps(out), flush=True)


def shrink_sweep(args, wl):
    """Every feasible configuration of the standalone down-projection on this workload, timed
    (microseconds per launch, HIP events, median of three batches of 20): the bf16-MFMA tile
    family against the wave-reduction (BGMV) kernel, with the library's default launch
    (lora_shrink) beside them.  Each configuration's t is checked against lora_shrink's."""
    import torch
    import precision_gemm_amd as P
    from precision_gemm_amd import tune
    from workloads.device import upload
    x, w, ad, ids = upload(wl)
    seg = P.build_segments(ids, ad.n)
    ref = P.shrink(x, seg, ad)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t = torch.empty_like(ref)

    def timed(fn, reps=20):
        fn()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        return sorted(times)[1]

    def info(tg, jp, u, m):
        try:
            return P.shrink_config_info(tg, jp, u, nt=m)
        except Exception:
            return None
    default_us = timed(lambda: P.shrink(x, seg, ad, t=t))
    rows = []
    for node in tune.space():
        if not tune.feasible(node, info, wl.T):
            continue
        cfg = tune.to_config(node)
        us = timed(lambda: P.shrink_configured(x, seg, ad, cfg, t=t))
        d = float((t - ref).norm() / ref.norm())
        rows.append((node, cfg, us, d))
    names = ("TG", "JP", "U", "TBLK", "ORDER")
    fam = lambda tg: "wave_reduction" if tg == 0 else "mfma"  # noqa: E731
    out = {"workload": args.workload, "what": "standalone down-projection, us per launch (HIP events)",
           "default_us": default_us, "kernel_sha": kernel_source_sha(), "configurations": len(rows)}
    for f in ("mfma", "wave_reduction"):
        sub = [r for r in rows if fam(r[0][0]) == f]
        if sub:
            b = min(sub, key=lambda r: r[2])
            out[f] = {"best": dict(zip(names, b[1])), "best_us": b[2], "max_rel_frob_vs_default": max(r[3] for r in sub),
                      "all": [[list(r[1]), round(r[2], 3)] for r in sorted(sub, key=lambda r: r[2])]}
    print(json.dumps(out), flush=True)


def ablation_merged(args, wl):
    """The per-token merged-weight formulation against the fused layer (both with x in bf16:
    by the merged-weight identity they compute the same layer), microseconds per call from
    HIP events around a graph of K calls, and both checked against the oracle on sampled rows."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from oracle.layer import LowpWeight, layer
    x, w, ad, ids = upload(wl)
    wr = P.LowpWeight(wl.fmt, torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda())
    rows, ptrs = P.adapter_rows(ad)
    seg = P.build_segments(ids, ad.n)
    ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max)
    y_m = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    y_f = torch.empty_like(y_m)
    calls = {"merged": lambda: P.merged_layer(x, wr, ids, ad, ptrs, y=y_m),
             "fused_act_bf16": lambda: P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, fuse_shrink=True, y=y_f,
                                                                 act_bf16=True)}
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / args.steps
    rows_chk = np.arange(wl.T) if wl.T <= 256 else np.linspace(0, wl.T - 1, 64).astype(int)
    ref = layer(wl.x[rows_chk], LowpWeight(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale,
                np.asarray(wl.ids)[rows_chk], act="bf16")["y"]
    parity = {}
    for name, yy in (("merged", y_m), ("fused_act_bf16", y_f)):
        d = yy.float().cpu().numpy().astype(np.float64)[rows_chk] - ref
        parity[name] = {"max_rel": float(np.abs(d).max() / np.abs(ref).max()),
                        "frob_rel": float(np.linalg.norm(d) / np.linalg.norm(ref))}
    out = {"workload": args.workload, "what": "us per layer call, graph of K calls, HIP events",
           "merged_us": res["merged"], "fused_act_bf16_us": res["fused_act_bf16"],
           "merged_over_fused": res["merged"] / res["fused_act_bf16"], "adapters_present": int(len(np.unique(wl.ids))),
           "parity": parity, "steps": args.steps, "kernel_sha": kernel_source_sha()}
    print(json.dumps(out), flush=True)


def backward_flops(wl):
    """Algorithmic FLOPs of one backward call: dX = dY W_d^T (2TKN) and, per token, the
    adapter products u = dY B_a^T, s u A_a^T, and its shares of dA_a and dB_a (2 r_a each of
    N, K, K, N)."""
    r_tok = wl.ranks[np.asarray(wl.ids)]
    return 2.0 * wl.T * wl.K * wl.N + float(np.sum(4.0 * r_tok * (wl.K + wl.N)))


def backward_bytes(wl):
    """Algorithmic bytes of one backward call: x, dY and dX in bf16 (T K, T N, T K), the 8-bit
    W^T codes and their channel scales (N K + 4 N), u and the forward t in fp32 (2 T r_max), and
    per adapter present B_a and A_a in bf16 (2 r_a (N + K) each) and dA_a, dB_a in fp32
    (4 r_a (K + N) each)."""
    present = sorted(set(int(a) for a in np.asarray(wl.ids)))
    r_max = int(max(wl.ranks))
    per_ad = sum(6.0 * int(wl.ranks[a]) * (wl.K + wl.N) for a in present)
    return (2.0 * wl.T * (2 * wl.K + wl.N) + wl.N * wl.K + 4.0 * wl.N + 8.0 * wl.T * r_max + per_ad)


def backward(args, wl):
    """A step is one lora_backward call (u, dA and dB, dX) on the workload's batch with a
    seeded dY; K calls in one HIP graph, timed with HIP events on the launch stream; two input
    sets alternate.  Parity of dX on sampled rows against the backward oracle."""
    import torch
    import precision_gemm_amd as P
    import workloads
    from workloads.device import bf16_tensor, upload
    from oracle import backward as BW
    from oracle.layer import LowpWeight as OW
    if wl.fmt != "fp8":
        print(json.dumps({"error": "the backward runs on an FP8 base only"}))
        sys.exit(2)
    dy_bits = workloads.grad_output(wl.T, wl.N, wl.seed + 1000)
    S = []
    for _ in range(2):
        x, w, ad, ids = upload(wl)
        q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda()
        sc = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda()
        wt = P.pack_weight_t(P.LowpWeight("fp8", q, sc))
        del q
        bw = P.pack_adapters_bwd(ad)
        seg = P.build_segments(ids, ad.n)
        t = P.shrink(x, seg, ad)                       # the forward's down-projection
        dy = bf16_tensor(dy_bits)
        dx = torch.empty((wl.T, wl.K), dtype=torch.bfloat16, device="cuda")
        u = torch.empty((wl.T, ad.r_max), dtype=torch.float32, device="cuda")
        S.append(dict(x=x, dy=dy, t=t, wt=wt, sc=sc, seg=seg, ad=ad, bw=bw, dx=dx, u=u,
                      grads=P.alloc_grads(ad, wl.K, wl.N)))
    torch.cuda.synchronize()

    def step(i):
        d = S[i % 2]
        P.lora_backward(d["x"], d["dy"], d["t"], d["wt"], d["sc"], d["seg"], d["ad"], d["bw"], dx=d["dx"],
                        u=d["u"], grads=d["grads"])

    step(0)
    torch.cuda.synchronize()
    rows = np.arange(wl.T) if wl.T <= 256 else np.linspace(0, wl.T - 1, 128).astype(int)
    ref = BW.lora_backward(wl.x[rows], OW(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale,
                           np.asarray(wl.ids)[rows], dy_bits[rows])
    dxg = S[0]["dx"].float().cpu().numpy().astype(np.float64)[rows]
    dlt = dxg - ref["dx"]
    parity = {"dx_max_rel": float(np.abs(dlt).max() / np.abs(ref["dx"]).max()),
              "dx_frob_rel": float(np.linalg.norm(dlt) / np.linalg.norm(ref["dx"])), "rows_checked": int(len(rows))}
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
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
    total_s = time.perf_counter() - t0
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1e3 / K
    flops = backward_flops(wl)
    achieved = flops / (call_us * 1e-6) / 1e12
    out = {
        "metric": "µs per LoRA backward call (dX, dA, dB) and MFMA TFLOP/s", "value": round(total_s * 1e6 / K, 3),
        "unit": "us/call", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": total_s * 1e3 / K,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16xfp8", "data": "synthetic",
        "config": {"workload": args.workload + "_backward", "T": wl.T, "K": wl.K, "N": wl.N, "w_format": wl.fmt,
                   "adapters": wl.n_adapters, "ranks": sorted(set(int(r) for r in wl.ranks)),
                   "timing": "hip graph of K steps"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": stored_traffic(args.workload + "_backward", kernel_source_sha()), "call_us": call_us,
                     "per_call_flops": flops, "per_call_bytes": backward_bytes(wl),
                     "kernel": "backward call: down-projection of dY (u) + k_bwd_grad (dA, dB) + k_bwd_dx"},
        "parity": parity, "kernel_sha": kernel_source_sha(),
    }
    if args.copy_mb > 0:  # counter calibration: three device copies of known size after the timed region
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
        sub = np.arange(wl.T) if wl.T <= 256 else np.linspace(0, wl.T - 1, 512).astype(int)
        runs, c0 = 0, time.perf_counter()
        while True:
            BW.lora_backward(wl.x[sub], OW(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale, np.asarray(wl.ids)[sub],
                             dy_bits[sub])
            runs += 1
            el = time.perf_counter() - c0
            if el >= 12.0 or runs >= 1000:
                break
        out["cpu_baseline"] = {"value": el / runs * (wl.T / len(sub)) * 1e6, "unit": "us/call", "cores": int(cores),
                               "kind": "oracle",
                               "sample": f"{runs} backward oracle run(s) on {len(sub)} of {wl.T} tokens, scaled by "
                                         f"T/{len(sub)} ({el:.1f} s)"}
    print(json.dumps(out), flush=True)


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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill",
                    choices=["tiny", "decode_qkv", "decode_gateup", "prefill", "downproj_fp4", "decoder_layer"])
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0: enough for 2x 256 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--act", choices=["mxfp8", "bf16"], default="mxfp8",
                    help="activations of the base product: MXFP8 (default) or bf16 as they are")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--tune-shrink", type=int, default=0, metavar="STEPS",
                    help="instead of the layer call: search the down-projection's configurations for the "
                         "workload (STEPS steps of the stochastic search) and print the result")
    ap.add_argument("--ablation-merged", action="store_true",
                    help="instead of the layer call: time the per-token merged-weight layer (lora_merged_layer) "
                         "against the fused layer with 16-bit activations on the workload")
    ap.add_argument("--shrink-sweep", action="store_true",
                    help="instead of the layer call: time every feasible configuration of the standalone "
                         "down-projection (MFMA tiles and wave reductions) on the workload")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the layer call: time the backward (lora_backward) on the workload (FP8 base)")
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
    if args.tune_shrink:
        tune_shrink(args, wl)
        return
    if args.ablation_merged:
        ablation_merged(args, wl)
        return
    if args.backward:
        backward(args, wl)
        return
    if args.shrink_sweep:
        shrink_sweep(args, wl)
        return
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

    # The timed unit is the layer call on a batch whose segments are built: in a serving
    # engine one segment build serves every LoRA layer of a step.  The builder is timed on its
    # own, and the call that also builds the segments (LORA_BUILD_SEGMENTS, as the first LoRA
    # layer of a batch runs it) is reported beside it as "all in".
    for d in S:
        P.build_segments(d["ids"], d["ad"].n, out=d["seg"])
    torch.cuda.synchronize()

    def step(s):
        d = S[s % sets]
        P.gemm_lowp_lora_epilogue(d["x"], d["w"], d["seg"], d["ad"], d["ws"], fuse_shrink=True, y=d["y"],
                                  act_bf16=a16)

    def step_all_in(s):
        d = S[s % sets]
        P.gemm_lowp_lora_epilogue(d["x"], d["w"], d["seg"], d["ad"], d["ws"], fuse_shrink=True, y=d["y"],
                                  build_segments=True, act_bf16=a16)

    def builder(s):
        d = S[s % sets]
        P.build_segments(d["ids"], d["ad"].n, out=d["seg"])

    # parity of the benchmarked call against the oracle (whole layer for decode shapes)
    step(0)
    torch.cuda.synchronize()
    parity = None
    try:
        from oracle.layer import LowpWeight, layer
        if wl.T <= 256:
            rows = np.arange(wl.T)
        else:  # 128 evenly spaced rows plus the first and the last row of every segment
            rows = set(np.linspace(0, wl.T - 1, 128).astype(int).tolist())
            for a in np.unique(wl.ids):
                where = np.flatnonzero(np.asarray(wl.ids) == a)
                rows.update([int(where[0]), int(where[-1])])
            rows = np.array(sorted(rows))
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
        call_us = all_in_us = builder_us = None
    else:
        # K whole steps in one graph, timed from the host
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for i in range(K):
                step(i)
        # the same with the segments built in the call, and the builder alone
        g_allin = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_allin):
            for i in range(K):
                step_all_in(i)
        g_build = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_build):
            for i in range(K):
                builder(i)
        g_all.replay()
        g_allin.replay()
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

        call_us = event_us(g_all)        # the whole layer call: its pre-pass (if any) and layer kernel
        all_in_us = event_us(g_allin)    # the same, building the segments too
        builder_us = event_us(g_build)   # the segment builder alone
    # every workspace must report a clean status
    status = max(P.workspace_status(d["ws"]) for d in S)

    us_per_step = total_s * 1e6 / K
    dom_us = call_us if call_us is not None else us_per_step
    prefill = wl.T > 256
    peak = (BF16_PEAK_TFLOPS if a16 else FP8_PEAK_TFLOPS) if prefill else HBM_PEAK_GBS

    def rate(us):
        return flops / (us * 1e-6) / 1e12 if prefill else nbytes / (us * 1e-6) / 1e9

    achieved = rate(dom_us)
    roof = {"bound": "mfma" if prefill else "hbm", "achieved": achieved, "peak": peak,
            "unit": "TFLOP/s" if prefill else "GB/s", "frac": achieved / peak}
    sha = kernel_source_sha()
    tag = args.workload + ("_act_bf16" if a16 else "")
    roof["traffic"] = stored_traffic(tag, sha)
    a16_rows = a16 and wl.T > 128 and wl.fmt == "fp8" and wl.N % 256 == 0
    roof["kernel"] = ("layer call: k_prep_rows (down-projection, plain t) + k_gemm_a16 (64 x 256 tiles, "
                      "bf16-MFMA GEMM on widened W + LoRA epilogue)" if a16_rows else
                      "layer call: k_layer (down-projection + bf16-MFMA GEMM on widened W + LoRA epilogue)"
                      if a16 else "layer call: MXFP8 pre-pass above 16 tokens (with the down-projection above 128 "
                      "tokens) + k_layer (scaled-MFMA GEMM + LoRA epilogue; down-projection in the same launch up "
                      "to 128 tokens)")
    roof["per_call_bytes"] = nbytes
    roof["per_call_flops"] = flops
    roof["call_us"] = dom_us
    if all_in_us is not None:
        roof["all_in"] = {"what": "the call also builds the segments (LORA_BUILD_SEGMENTS)", "us": all_in_us,
                          "achieved": rate(all_in_us), "frac": rate(all_in_us) / peak}

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
        "all_in_us": all_in_us,
        "builder_us": builder_us,
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
