"""Shared helpers for the GPU tests: run the HIP path through the C ABI and compare it
with the oracle.  The oracle side only ever sees the generated numpy inputs."""

from __future__ import annotations

import functools

import numpy as np

import workloads
from oracle.layer import LowpWeight as OracleWeight, layer as oracle_layer

# tolerances fixed for the layer output (max error relative to max |y_ref|, relative
# Frobenius error) and for the down-projection t (relative Frobenius)
Y_MAX_REL = 1e-2
Y_FROB_REL = 5e-3
T_FROB_REL = 1e-4


@functools.lru_cache(maxsize=8)
def named(name: str):
    return workloads.make(name)


@functools.lru_cache(maxsize=8)
def named_oracle(name: str, rows: tuple | None = None):
    wl = named(name)
    return run_oracle(wl, rows)


def sample_rows(wl, n: int, seed: int) -> tuple:
    """Rows for an oracle check of a long batch (every row of y depends only on its own
    token): n random rows plus the first and the last row of every adapter's segment in
    token order, so that the shortest segments are always checked."""
    ids = np.asarray(wl.ids)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(wl.T, n, replace=False).tolist())
    for a in np.unique(ids):
        where = np.flatnonzero(ids == a)
        rows.update([int(where[0]), int(where[-1])])
    return tuple(sorted(rows))


def run_oracle(wl, rows=None, act="mxfp8"):
    ids = np.asarray(wl.ids)
    x = wl.x
    if rows is not None:
        rows = np.asarray(rows)
        x, ids = x[rows], ids[rows]
    return oracle_layer(x, OracleWeight(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale, ids, act=act)


def bf16_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(y: np.ndarray, y_ref: np.ndarray):
    d = y - y_ref
    max_rel = np.abs(d).max() / max(np.abs(y_ref).max(), 1e-300)
    frob = np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-300)
    return float(max_rel), float(frob)


def assert_y_close(y, y_ref, what=""):
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    m, f = errors(y, y_ref)
    assert m <= Y_MAX_REL and f <= Y_FROB_REL, f"{what}: max_rel={m:.3e} frob={f:.3e}"
    return m, f


def assert_t_close(t, t_ref, what=""):
    f = np.linalg.norm(t - t_ref) / max(np.linalg.norm(t_ref), 1e-300)
    assert f <= T_FROB_REL, f"{what}: t frob={f:.3e}"
    return f


def run_gpu(wl, *, fused=True, want_t=True, base_only=False, build=False, act_bf16=False):
    """Run the layer on the GPU; returns dict of numpy results.  build: the fused layer
    call also builds the segments (no separate segment launch); act_bf16: the base
    product on the bf16 activations as they are."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    x, w, ad, ids = upload(wl)
    ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max)
    out = {}
    seg = P.empty_segments(ids, ad.n) if build else P.build_segments(ids, ad.n)
    if build:
        seg.seg_indptr.fill_(-7)
        seg.sorted_tok.fill_(-7)
        t = torch.empty((wl.T, ad.r_max), dtype=torch.float32, device="cuda") if want_t else None
        y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=t, fuse_shrink=True, build_segments=True,
                                      act_bf16=act_bf16)
        if t is not None:
            out["t"] = t
        torch.cuda.synchronize()
        seg.err.fill_(P.workspace_segment_error(ws))
    elif base_only:
        y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=None, fuse_shrink=False, act_bf16=act_bf16)
    elif fused:
        t = torch.empty((wl.T, ad.r_max), dtype=torch.float32, device="cuda") if want_t else None
        y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=t, fuse_shrink=True, act_bf16=act_bf16)
        if t is not None:
            out["t"] = t
    else:
        t = P.shrink(x, seg, ad, ws)
        y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=t, fuse_shrink=False, act_bf16=act_bf16)
        out["t"] = t
    torch.cuda.synchronize()
    out["status"] = P.workspace_status(ws)
    res = {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()}
    res["y"] = bf16_to_f64(y)
    res["y_bits"] = y.view(torch.int16).cpu().numpy()
    res["seg_indptr"] = seg.seg_indptr.cpu().numpy()
    res["sorted_tok"] = seg.sorted_tok.cpu().numpy()
    res["err"] = int(seg.err.item())
    return res
